// Two-GEMM cascade whose second GEMM runs on gfx950's fp8 matrix instruction
// (v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 operands and unit scales): the
// first GEMM is fp16 or bf16 on the 32x32x16 instruction, its fp32 result is
// rounded to fp8 on chip and becomes the second GEMM's operand.
//
// Page 1 derives the rearrangement from the register layouts of the result
// of one instruction and the operand of the next, per data type; here they
// are of different instructions and types.  The fp8 instruction takes 32
// values per lane: lane l holds row l%32 and 32 k-slots, the two 32-lane
// halves holding different slots, and the A and B operands pair their slots
// the same way (checked on the hardware by b2b_mfma_probe).  The first GEMM
// is computed transposed, so lane (m = l%32, h = l/32) holds 16 values of
// row m of the intermediate per 32-column result tile (columns 8a + 4h +
// 0..3, registers 4a..4a+3).  Relabelled: K-step j of the second GEMM takes
// result tiles 2j and 2j+1, slot u of lane half h holding intermediate column
//     64j + 32(u/16) + 8((u%16)/4) + 4h + u%4
// (result register u%16 of tile 2j + u/16) -- nothing moves between lanes.
// B1 is staged in LDS in that K order, one 16-byte piece per lane and half
// of the slots, so a weight fragment is two conflict-free 16-byte reads.
#pragma once
#include "kernels_gen.hpp"

namespace b2bk {

typedef int i8v_t __attribute__((ext_vector_type(8)));

// DT0_: type of A, B0 and the first GEMM (DT_F16 / DT_BF16); DTD_: type of D;
// MAXD_: bound on K, N1, N2; PF_: A tiles fetched ahead (0 or 1); WAVES_: 8
// (256-row tiles) or 4 (128-row tiles, two workgroups a CU where LDS allows).
// The members are those the 32x32x16 run-time-width building blocks read.
template <int DT0_, int DTD_, int MAXD_, int PF_, int WAVES_ = 8>
struct F8Cfg {
    static constexpr int DT = DT0_, DTD = DTD_, NST = 2, MAXD = MAXD_, MODE = MODE_RELABEL, PF = PF_;
    static constexpr bool RTM = false;   // types fixed at compile time
    static constexpr bool TAIL = false;  // widths whole granules
    static constexpr int WAVES = WAVES_, THREADS = 64 * WAVES, ROWS_WAVE = 32, ROWS_WG = ROWS_WAVE * WAVES;
    static constexpr int MKS = MAXD / 16, MNT = MAXD / 32, MKS8 = MAXD / 64;
    static constexpr int LDS_MAX = 160 * 1024;
    static constexpr int stype(int s) { return s == 0 ? DT : DTD; }   // s == 2: D (the fp8 stage is not 16-bit)
    static_assert(DT != DT_F64 && DTD != DT_F64 && MAXD % 64 == 0 && (PF == 0 || PF == 1), "config");
    // the 16-bit weights (B0 alone) for gen_stage_weights
    struct Stage0 {
        static constexpr int NST = 1, WAVES = WAVES_, THREADS = 64 * WAVES_;
    };
};

// LDS bytes: B0 (16-bit), B1 (fp8), then 4 KB of D staging per wave when it fits
__host__ __device__ inline int64_t f8_weight_bytes(const int32_t* d) {
    return (int64_t)d[0] * d[1] * 2 + (int64_t)d[1] * d[2];
}
__host__ __device__ inline bool f8_stage_d(const int32_t* d, int waves = 8) {
    return f8_weight_bytes(d) + waves * 4096 <= 160 * 1024;
}
__host__ __device__ inline int64_t f8_lds_bytes(const int32_t* d, int waves = 8) {
    return f8_weight_bytes(d) + (f8_stage_d(d, waves) ? waves * 4096 : 0);
}

// fp8 x fp8 -> fp32 on the 32x32x64 instruction, E4M3 operands, scales 2^0
__device__ __forceinline__ f16x_t f8_mma(const i8v_t& a, const i8v_t& b, const f16x_t& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// result tiles 2j (acc0) and 2j+1 (acc1) -> fp8 operand of K-step j (slots
// 0-15 from acc0's registers 0-15, 16-31 from acc1's)
__device__ __forceinline__ i8v_t f8_operand(const f16x_t& acc0, const f16x_t& acc1) {
    i8v_t o;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        o[d] = f8_pack4(acc0[4 * d], acc0[4 * d + 1], acc0[4 * d + 2], acc0[4 * d + 3]);
        o[4 + d] = f8_pack4(acc1[4 * d], acc1[4 * d + 1], acc1[4 * d + 2], acc1[4 * d + 3]);
    }
    return o;
}

// B1 fragment (32-column output tile t, K-step j): lane l's slots 16q..16q+15
// at off + ((t * ks8 + j) * 2 + q) * 1024 + 16 l
__device__ __forceinline__ i8v_t f8_wfrag(const unsigned char* lds, int off, int ks8, int t, int j, int lane) {
    const unsigned char* p = lds + off + (t * ks8 + j) * 2048 + lane * 16;
    const u4_t lo = *(const u4_t*)p, hi = *(const u4_t*)(p + 1024);
    return i8v_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// B1 (fp8, n1 x n2, row-major with leading dimension ldb bytes) of batch b ->
// LDS fragments in the relabelled K order: piece (t, j, q, lane (n', h))
// gathers rows 64j + 32q + 8(i/4) + 4h + i%4 (i < 16) of column 32t + n'.
template <class C, int S = 1>
__device__ inline void f8_stage_b1(unsigned char* lds, int off, const KArgs& args, int b, int n1, int n2) {
    const auto rs = make_rsrc((const char*)args.B[S] + (int64_t)b * args.sB[S], (uint32_t)(n1 * args.ldb[S]));
    const int ks8 = n1 / 64, pieces = (n2 / 32) * ks8 * 2 * 64;
    for (int p = (int)threadIdx.x; p < pieces; p += C::THREADS) {
        const int lane = p & 63, q = (p >> 6) & 1, tj = p >> 7;
        const int t = tj / ks8, j = tj % ks8;
        const int col = 32 * t + (lane & 31), h = lane >> 5;
        unsigned w[4] = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int row = 64 * j + 32 * q + 8 * (i >> 2) + 4 * h + (i & 3);
            const unsigned v = __builtin_amdgcn_raw_buffer_load_b8(rs, row * (int)args.ldb[S] + col, 0, 0);
            w[i >> 2] |= v << (8 * (i & 3));
        }
        *(u4_t*)(lds + off + tj * 2048 + q * 1024 + lane * 16) = u4_t{w[0], w[1], w[2], w[3]};
    }
}

template <class C>
__device__ __forceinline__ void f8_body(const KArgs& args) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int d0 = args.dims[0], d1 = args.dims[1], d2 = args.dims[2];
    GenMat m0[1];
    m0[0].init(0, d0, d1);
    const int off1 = d0 * d1 * 2;                       // B1 fragments follow B0
    const int32_t dd[3] = {d0, d1, d2};
    const int stg = f8_stage_d(dd, C::WAVES) ? off1 + d1 * d2 + wave * 4096 : -1;
    GenFrag fr0;
    fr0.init(m0[0], false, lane);
    const int ks0 = d0 / 16, ks8 = d1 / 64, nt2 = d2 / 32;

    TileRange<C::ROWS_WG, C::ROWS_WAVE> tr;
    if (!tr.init(args, wave)) return;
    // Up to 128 wide the first segment's B0 copies go out before the entry
    // arithmetic and the first A tile before B1's gather.  At 256 a tile of A
    // is 128 KB a CU: ahead of the gather's byte loads in the memory pipeline
    // it slows the gather more than the overlap gains (2-3 %), so there B0 is
    // staged through registers and A follows the weights.
    constexpr bool EARLY = C::MAXD <= 128;
    if constexpr (EARLY) gen_copy_weights<typename C::Stage0>(lds, m0, args, tr.t0 / tr.TB, wave);
    __builtin_amdgcn_sched_barrier(0);
    auto a_rsrc = [&](int t) { return tr.a_rsrc(args.A, args.lda, args.sA, 2, t); };

    auto process = [&](int t, const u4_t (&a_in)[C::MKS]) __attribute__((always_inline)) {
        u4_t a[C::MKS];
#pragma unroll
        for (int j = 0; j < C::MKS; ++j) a[j] = a_in[j];
        gen_arrange_a<C>(a);
        const auto d_rs = tr.rsrc(args.D, args.ldd, args.sD, 2, t);
        // first GEMM: result tiles in pairs, each pair one fp8 K-step
        i8v_t x8[C::MKS8];
        gen_gemm<C, C::DT>(lds, fr0, a, ks0, d1 / 32,
                           [&](int tt, const f16x_t& a0, const f16x_t& a1, bool) __attribute__((always_inline)) {
                               x8[tt / 2] = f8_operand(a0, a1);
                           });
        // second GEMM on the fp8 instruction, output tiles in pairs
        const int nt2u = uniform_here(nt2), ks8u = uniform_here(ks8);
#pragma unroll
        for (int t2 = 0; t2 < C::MNT; t2 += 2) {
            if (t2 < nt2u) {
                const bool two = t2 + 1 < nt2u;
                const int t2b = two ? t2 + 1 : t2;
                // K-step 0 always exists: its products start from zero
                f16x_t acc0 = f8_mma(f8_wfrag(lds, off1, ks8u, t2, 0, lane), x8[0], f16x_t{});
                f16x_t acc1 = f8_mma(f8_wfrag(lds, off1, ks8u, t2b, 0, lane), x8[0], f16x_t{});
#pragma unroll
                for (int j = 1; j < C::MKS8; ++j)
                    if (j < ks8u) {
                        acc0 = f8_mma(f8_wfrag(lds, off1, ks8u, t2, j, lane), x8[j], acc0);
                        acc1 = f8_mma(f8_wfrag(lds, off1, ks8u, t2b, j, lane), x8[j], acc1);
                    }
                gen_store_pair<C>(lds, stg, acc0, acc1, two, d_rs, args.ldd, 32 * t2, lane);
            }
        }
    };

    const auto no_rsrc = make_rsrc(args.A, 0u);
    u4_t ring[C::PF + 1][C::MKS];
    int t = tr.t0;
    bool issued = EARLY;   // the first segment's B0 is on its way
    while (t < tr.t1) {
        const int b = t / tr.TB;
        tr.segment(t);
        if constexpr (EARLY) {
            if (!issued) {
                __syncthreads();   // the previous segment's weight reads are over
                gen_copy_weights<typename C::Stage0>(lds, m0, args, b, wave);
            }
            issued = false;
            // the first A tile, then B1's gather (its LDS writes wait for its
            // loads, and so, in order, for everything before them); then all
            // of it, the copies included, before the barrier
            gen_load_a<C>(ring[0], a_rsrc(t), no_rsrc, args.lda, ks0, lane);
            f8_stage_b1<C>(lds, off1, args, b, d1, d2);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        } else {
            __syncthreads();   // the previous segment's weight reads are over
            gen_stage_weights<typename C::Stage0>(lds, m0, args, b);
            f8_stage_b1<C>(lds, off1, args, b, d1, d2);
            __syncthreads();
            gen_load_a<C>(ring[0], a_rsrc(t), no_rsrc, args.lda, ks0, lane);
        }
        if constexpr (C::PF == 0) {
            for (;;) {
                process(t, ring[0]);
                if (++t >= tr.t_end) break;
                gen_load_a<C>(ring[0], a_rsrc(t), no_rsrc, args.lda, ks0, lane);
            }
        } else {
            for (;;) {
                gen_load_a<C>(ring[1], a_rsrc(t + 1), no_rsrc, args.lda, ks0, lane);
                process(t, ring[0]);
                if (++t >= tr.t_end) break;
                gen_load_a<C>(ring[0], a_rsrc(t + 1), no_rsrc, args.lda, ks0, lane);
                process(t, ring[1]);
                if (++t >= tr.t_end) break;
            }
        }
    }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void f8_kernel(KArgs args) {
    f8_body<C>(args);
}

// The second kernel of the unfused comparison of such a cascade: one GEMM of
// an fp8 A (the intermediate the first kernel wrote as E4M3 bytes) and an fp8
// B on the fp8 instruction, D in DTD_.  A is read in the relabelled slot
// order of the fused kernel: dword 4q + i of K-step j holds bytes 64j + 32q +
// 8i + 4(l/32) + 0..3 of row l%32.  K a multiple of 64, N of 32.
template <int DTD_, int MAXD_>
struct F8ACfg {
    static constexpr int DT = DT_F16, DTD = DTD_, NST = 1, MAXD = MAXD_, MODE = MODE_RELABEL, PF = 1;
    static constexpr bool RTM = false;   // types fixed at compile time
    static constexpr bool TAIL = false;  // widths whole granules
    static constexpr int WAVES = 8, THREADS = 64 * WAVES, ROWS_WAVE = 32, ROWS_WG = ROWS_WAVE * WAVES;
    static constexpr int MKS = MAXD / 16, MNT = MAXD / 32, MKS8 = MAXD / 64;
    static constexpr int LDS_MAX = 160 * 1024;
    static constexpr int stype(int) { return DTD; }   // D, for gen_store_pair
    static_assert(MAXD % 64 == 0, "config");
};

// LDS bytes: the fp8 weights, then 4 KB of D staging per wave when it fits
__host__ __device__ inline int64_t f8a_lds_bytes(const int32_t* d) {
    const int64_t w = (int64_t)d[0] * d[1];
    return w + (w + 8 * 4096 <= 160 * 1024 ? 8 * 4096 : 0);
}

template <class C>
__device__ __forceinline__ void f8a_load(i8v_t (&x)[C::MKS8], __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t none,
                                         int64_t lda, int ks8, int lane) {
    const int m = lane & 31, h = lane >> 5;
#pragma unroll
    for (int j = 0; j < C::MKS8; ++j) {
        const auto src = j < ks8 ? rs : none;
#pragma unroll
        for (int d = 0; d < 8; ++d)
            x[j][d] = __builtin_amdgcn_raw_buffer_load_b32(
                src, (int)(m * lda + 64 * j + 32 * (d >> 2) + 8 * (d & 3) + 4 * h), 0, 0);
    }
}

template <class C>
__device__ __forceinline__ void f8a_body(const KArgs& args) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int d0 = args.dims[0], d1 = args.dims[1];
    const int stg = (int64_t)d0 * d1 + 8 * 4096 <= 160 * 1024 ? d0 * d1 + wave * 4096 : -1;
    const int ks8 = d0 / 64, nt = d1 / 32;

    TileRange<C::ROWS_WG, C::ROWS_WAVE> tr;
    if (!tr.init(args, wave)) return;
    auto a_rsrc = [&](int t) { return tr.a_rsrc(args.A, args.lda, args.sA, 1, t); };
    auto process = [&](int t, const i8v_t (&x)[C::MKS8]) __attribute__((always_inline)) {
        const auto d_rs = tr.rsrc(args.D, args.ldd, args.sD, 2, t);
        const int ntu = uniform_here(nt), ks8u = uniform_here(ks8);
#pragma unroll
        for (int t2 = 0; t2 < C::MNT; t2 += 2) {
            if (t2 < ntu) {
                const bool two = t2 + 1 < ntu;
                const int t2b = two ? t2 + 1 : t2;
                // K-step 0 always exists: its products start from zero
                f16x_t acc0 = f8_mma(f8_wfrag(lds, 0, ks8u, t2, 0, lane), x[0], f16x_t{});
                f16x_t acc1 = f8_mma(f8_wfrag(lds, 0, ks8u, t2b, 0, lane), x[0], f16x_t{});
#pragma unroll
                for (int j = 1; j < C::MKS8; ++j)
                    if (j < ks8u) {
                        acc0 = f8_mma(f8_wfrag(lds, 0, ks8u, t2, j, lane), x[j], acc0);
                        acc1 = f8_mma(f8_wfrag(lds, 0, ks8u, t2b, j, lane), x[j], acc1);
                    }
                gen_store_pair<C>(lds, stg, acc0, acc1, two, d_rs, args.ldd, 32 * t2, lane);
            }
        }
    };

    const auto no_rsrc = make_rsrc(args.A, 0u);
    i8v_t ring[2][C::MKS8];
    int t = tr.t0;
    while (t < tr.t1) {
        const int b = t / tr.TB;
        tr.segment(t);
        __syncthreads();   // the previous segment's weight reads are over
        f8_stage_b1<C, 0>(lds, 0, args, b, d0, d1);
        __syncthreads();
        f8a_load<C>(ring[0], a_rsrc(t), no_rsrc, args.lda, ks8, lane);
        for (;;) {
            f8a_load<C>(ring[1], a_rsrc(t + 1), no_rsrc, args.lda, ks8, lane);
            process(t, ring[0]);
            if (++t >= tr.t_end) break;
            f8a_load<C>(ring[0], a_rsrc(t + 1), no_rsrc, args.lda, ks8, lane);
            process(t, ring[1]);
            if (++t >= tr.t_end) break;
        }
    }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void f8a_kernel(KArgs args) {
    f8a_body<C>(args);
}

// One fp8 instruction on raw operands (64 lanes x 32 E4M3 bytes each) and the
// conversion of 64 x 4 floats: probes of the operand pairing and the rounding.
template <int = 0>
__global__ __launch_bounds__(64) void mfma_f8_probe_kernel(const void* a, const void* b, void* c) {
    const int lane = threadIdx.x;
    const i8v_t av = ((const i8v_t*)a)[lane], bv = ((const i8v_t*)b)[lane];
    ((f16x_t*)c)[lane] = f8_mma(av, bv, f16x_t{});
}
template <int = 0>
__global__ __launch_bounds__(64) void cvt_f8_probe_kernel(const float* x, int* y) {
    const int lane = threadIdx.x;
    y[lane] = f8_pack4(x[4 * lane], x[4 * lane + 1], x[4 * lane + 2], x[4 * lane + 3]);
}

}  // namespace b2bk
