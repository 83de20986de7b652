// Device code of the fused cascaded GEMM for gfx950 (CDNA4).
//
// Page 1 ("数据处理方法、装置、设备及介质", detailed description) fuses GEMMs
// whose output feeds the next GEMM directly, so the intermediate never makes
// the round trip through memory; where the first GEMM's result layout in the
// registers differs from the layout the second GEMM needs, the result is
// rearranged in the registers (exchange rounds scheduled by the coordination
// matrix of Fig. 4) or through shared memory, then fed to the next GEMM.
//
// gfx950 realisation (one wave = 64 lanes):
//  * every GEMM is a chain of MFMA instructions: v_mfma_f32_16x16x32_{f16,bf16}
//    (float32 accumulation) or v_mfma_f64_16x16x4_f64;
//  * the first GEMM is computed transposed, C0^T = B0^T . A^T, so a lane's
//    accumulators hold (part of) one row of C0; that is the layout the next
//    GEMM's operand wants up to a move between 16-lane rows ("orientation T").
//    The plain orientation (C0 = A . B0, lanes hold columns) is kept as an
//    option for the coordination-matrix and LDS executors;
//  * the weights B0, B1 (, B2) of the current batch sit in LDS, stored in
//    fragment-major order so that every MFMA operand read is one contiguous
//    ds_read per lane;
//  * each wave streams a tile of 16*MT rows of A straight from HBM into
//    operand registers (16-byte loads, the next tile prefetched while the
//    current one computes), runs all stages, and writes its rows of D once;
//  * workgroups are persistent; consecutive tiles (hence mostly one batch,
//    one copy of its weights) go to workgroups on the same XCD.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

namespace b2bk {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef double d4_t __attribute__((ext_vector_type(4)));
typedef unsigned u4_t __attribute__((ext_vector_type(4)));
typedef unsigned u2_t __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1, DT_F64 = 2, DT_TF32 = 3 };
enum { MODE_BPERM = 1, MODE_PERMLANE = 2, MODE_LDS = 3, MODE_RELABEL = 4 };
// How the K index of a GEMM stage is laid over (K-step, lane group, slot).
enum {
    KM_NAT = 0,    // the MFMA's own order: k = KW*ks + (S)*g + u
    KM_PAIR64 = 1, // fp64 A read 16 bytes at a time: K-step 2j+e holds k = 8j + 2g + e
    KM_REL = 2     // k follows the previous stage's accumulator layout (no data movement)
};

constexpr int kMaxRounds = 8;
constexpr int kMaxStages = 8;       // GEMMs in one cascade

struct KArgs {
    const void* A;
    const void* B[kMaxStages];
    void* D;
    int64_t M;
    int64_t lda, ldb[kMaxStages], ldd;
    int64_t sA, sB[kMaxStages], sD; // batch strides, elements
    int32_t tiles_per_batch;
    int32_t total_tiles;
    int32_t dims[kMaxStages + 1];   // widths K, N1, N2, ... (kernels with run-time widths)
    int32_t tmask;                  // a 16-bit type per stage read at run time (bit s: bf16), where compiled so
    // coordination rounds per lane, p | give<<6 | r<<9: table 0 for the first
    // rearrangement (after GEMM0), table 1 for the later ones
    uint16_t sched[2][kMaxRounds][64];
};

// ---------------------------------------------------------------------------
// Element types
// ---------------------------------------------------------------------------
template <int DT> struct Ty;
template <> struct Ty<DT_F16> {
    using op_t = u4_t;
    using acc_t = f4_t;
    static constexpr int ELT = 2, KW = 32, FB = 16;
    __device__ static inline f4_t mma(u4_t a, u4_t b, f4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                      __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
    }
    // float32 -> binary16, round to nearest even (v_cvt_f16_f32), two per dword
    __device__ static inline unsigned pack(float x, float y) {
        h2_t v = {(_Float16)x, (_Float16)y};
        return __builtin_bit_cast(unsigned, v);
    }
};
template <> struct Ty<DT_BF16> {
    using op_t = u4_t;
    using acc_t = f4_t;
    static constexpr int ELT = 2, KW = 32, FB = 16;
    __device__ static inline f4_t mma(u4_t a, u4_t b, f4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf8_t, a),
                                                       __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
    }
    // float32 -> bfloat16, round to nearest even
    __device__ static inline unsigned pack(float x, float y) {
        bf2_t v = {(__bf16)x, (__bf16)y};
        return __builtin_bit_cast(unsigned, v);
    }
};
template <> struct Ty<DT_F64> {
    using op_t = double;
    using acc_t = d4_t;
    static constexpr int ELT = 8, KW = 4, FB = 8;
    __device__ static inline d4_t mma(double a, double b, d4_t c) {
        return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// Buffer resources: out-of-range loads return 0 and out-of-range stores are
// dropped, which masks the ragged last tile of M without branches.
// ---------------------------------------------------------------------------
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ inline u4_t ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}
__device__ inline u2_t ld64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
}
// Cache policy of D's stores: D is written once, so stores that write whole
// 128-byte row segments go non-temporal (nt) and do not displace the weights
// from the caches.  Stores that write parts of a line (D straight from the
// accumulator layout, the last chunk of a ragged row) keep the default
// policy, so that the L2 merges a line's pieces before writing it back: sent
// non-temporal, a line's pieces reached HBM separately (28 % more bytes
// written than D holds, on the tf32 three-GEMM kernel).  A's loads keep the
// default policy: non-temporal A loads measured no better on the two-GEMM
// fp16 workload and 1-3 % slower on the three-GEMM and fp64 ones.
constexpr int kStreamPolicy = 2;

// whole row segments of D
__device__ inline void st128(__amdgpu_buffer_rsrc_t r, uint32_t off, u4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, kStreamPolicy);
}
// a piece of a line of D
__device__ inline void st128_part(__amdgpu_buffer_rsrc_t r, uint32_t off, u4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ inline void st64(__amdgpu_buffer_rsrc_t r, uint32_t off, u2_t v) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}

__device__ inline u2_t dsplit(double d) { return __builtin_bit_cast(u2_t, d); }
__device__ inline double djoin(u2_t v) { return __builtin_bit_cast(double, v); }

// ---------------------------------------------------------------------------
// Cross-lane primitives
//  permlane32_swap(x, y): lanes 32..63 of x trade places with lanes 0..31 of y
//  permlane16_swap(x, y): odd 16-lane rows of x trade with even rows of y
// ---------------------------------------------------------------------------
__device__ inline void swap32(unsigned& x, unsigned& y) {
    auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    x = r[0];
    y = r[1];
}
__device__ inline void swap16(unsigned& x, unsigned& y) {
    auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    x = r[0];
    y = r[1];
}

// Two accumulator tiles of 16 columns, packed to 16-bit pairs (lane group g
// holds columns 4g..4g+3 of each: x0,x1 from the first tile, y0,y1 from the
// second) -> lane group g holds the 8 consecutive columns 8g..8g+7 as
// {x0, x1, y0, y1}.  Two rounds of row swaps: 32-lane halves, then 16-lane rows.
__device__ inline void regroup_pairs(unsigned& x0, unsigned& x1, unsigned& y0, unsigned& y1) {
    swap32(x0, y0);
    swap32(x1, y1);
    swap16(x0, y0);
    swap16(x1, y1);
}

// 4 x 4 transpose of 64-bit registers across the four 16-lane rows:
// afterwards register s of row g holds what register g of row s held.
__device__ inline void transpose_rows64(double (&r)[4]) {
    unsigned w[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u2_t v = dsplit(r[i]);
        w[0][i] = v[0];
        w[1][i] = v[1];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        swap32(w[h][0], w[h][2]);
        swap32(w[h][1], w[h][3]);
        swap16(w[h][0], w[h][1]);
        swap16(w[h][2], w[h][3]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = djoin(u2_t{w[0][i], w[1][i]});
}

// Coordination-matrix executor (Fig. 4): in round j every lane offers element
// give_j of its source registers and pulls, with one ds_bpermute, the value
// offered by lane p_j, which it files as its element r_j.  No lane is asked by
// two lanes in one round, so each round is a single permutation of the wave.
// Lane-dependent register choices are bitwise selects over values held in
// registers (vectors, never arrays in memory, so nothing is indexed
// dynamically and nothing goes to scratch).
template <int E> struct VecU;
template <> struct VecU<4> { typedef unsigned type __attribute__((ext_vector_type(4))); };
template <> struct VecU<8> { typedef unsigned type __attribute__((ext_vector_type(8))); };

template <int E>
__device__ inline typename VecU<E>::type exchange32(typename VecU<E>::type src,
                                                   typename VecU<E>::type code) {
    typename VecU<E>::type dst = {};
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const unsigned c = code[j];
        const unsigned give = 1u << ((c >> 6) & 7u), r = 1u << ((c >> 9) & 7u);
        unsigned v = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) v |= src[e] & (0u - ((give >> e) & 1u));
        const unsigned got = (unsigned)__builtin_amdgcn_ds_bpermute((int)((c & 63u) << 2), (int)v);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const unsigned m = 0u - ((r >> e) & 1u);
            dst[e] = (dst[e] & ~m) | (got & m);
        }
    }
    return dst;
}

// 64-bit elements: the same rounds, two ds_bpermute per round.
__device__ inline void exchange64(const double (&src)[4], double (&dst)[4], VecU<4>::type code) {
    VecU<8>::type s, d = {};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const u2_t w = dsplit(src[e]);
        s[2 * e] = w[0];
        s[2 * e + 1] = w[1];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const unsigned c = code[j];
        const unsigned give = 1u << ((c >> 6) & 7u), r = 1u << ((c >> 9) & 7u);
        unsigned lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned m = 0u - ((give >> e) & 1u);
            lo |= s[2 * e] & m;
            hi |= s[2 * e + 1] & m;
        }
        const int addr = (int)((c & 63u) << 2);
        const unsigned glo = (unsigned)__builtin_amdgcn_ds_bpermute(addr, (int)lo);
        const unsigned ghi = (unsigned)__builtin_amdgcn_ds_bpermute(addr, (int)hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const unsigned m = 0u - ((r >> e) & 1u);
            d[2 * e] = (d[2 * e] & ~m) | (glo & m);
            d[2 * e + 1] = (d[2 * e + 1] & ~m) | (ghi & m);
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = djoin(u2_t{d[2 * e], d[2 * e + 1]});
}

// Workgroup barrier with explicit waits: "s_waitcnt" for the given counts,
// then s_barrier.  The A ring and the weight chunks are written by buffer
// loads that go straight to LDS and complete through vmcnt, so the wait for
// the data needed next is written out (the loads behind it stay in flight);
// the asm also keeps the compiler from moving memory accesses across the
// barrier.
template <int N>
__device__ inline void barrier_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}
__device__ inline void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Barrier that first waits until at most `tiles` A tiles (L loads each) of
// this wave are still in flight; `tiles` is uniform, 0 <= tiles <= 4.
template <int L>
__device__ inline void barrier_tiles_in_flight(int tiles) {
    switch (tiles) {
        case 0: barrier_vm<0>(); break;
        case 1: barrier_vm<L>(); break;
        case 2: barrier_vm<2 * L>(); break;
        case 3: barrier_vm<3 * L>(); break;
        default: barrier_vm<4 * L>(); break;
    }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short tr4_t __attribute__((ext_vector_type(4)));

// Buffer load of 16 bytes per lane that writes LDS (lane i -> lds_dst + 16 i;
// lds_dst uniform).  Issued from inline asm so that the compiler does not add
// a full wait for it before every later LDS read (it cannot tell which LDS
// bytes are still in flight); the callers wait for it explicitly (vmcnt).
// M0 carries the LDS address; nothing else in these kernels keeps a value in
// M0 (no LDS-DMA builtins, no dynamic register indexing), so clobbering it,
// which the compiler warns about in general, is safe here.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool NT>
__device__ inline void lds_dma16(__amdgpu_buffer_rsrc_t rs, const unsigned char* lds_dst, int voff) {
    const unsigned a = (unsigned)(uintptr_t)(lds_ptr_t)lds_dst;
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                     : : "s"(a), "v"(voff), "s"(rs) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     : : "s"(a), "v"(voff), "s"(rs) : "memory", "m0");
}
#pragma clang diagnostic pop

// A wave-uniform count, made opaque where it is passed: the loops bounded by
// it then compare and branch on scalars at each step.  Otherwise the compiler
// evaluates every step's condition once, early, and keeps each result as a
// 64-bit lane mask in scalar registers, which run out and spill to vector
// lanes in the run-time-width kernels.
__device__ __forceinline__ int uniform_here(int x) {
    asm volatile("" : "+s"(x));
    return x;
}

// This lane's index, computed where it is called: the compiler can neither
// keep it (and the addresses derived from it) in a register across the
// kernel nor fold it into an earlier computation.
__device__ inline int lane_here() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

__device__ inline void wave_lds_fence() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Per-wave LDS scratch for the shared-memory rearrangement: 16 rows of one
// unit, row pitch padded by 16 bytes to spread the rows over the banks.
template <int DT> struct LdsRemap;
template <> struct LdsRemap<DT_F16> { static constexpr int PITCH = 32 * 2 + 16, BYTES = 16 * PITCH; };
template <> struct LdsRemap<DT_BF16> { static constexpr int PITCH = 32 * 2 + 16, BYTES = 16 * PITCH; };
template <> struct LdsRemap<DT_F64> { static constexpr int PITCH = 16 * 8 + 16, BYTES = 16 * PITCH; };

// ---------------------------------------------------------------------------
// 16-bit rearrangement of one unit (two accumulator tiles -> one K-step of 32)
// acc0/acc1: tiles 2c and 2c+1. Orientation T: lane (m = l%16, g = l/16) holds
// row m, columns 4g..4g+3 of each tile. Orientation N: lane holds column
// l%16, rows 4g..4g+3.  Result: lane holds row l%16, columns 8g..8g+7.
// ---------------------------------------------------------------------------
typedef VecU<8>::type code_t;

template <int DT, int MODE, bool ORN>
__device__ inline u4_t remap_unit16(f4_t acc0, f4_t acc1, code_t code, unsigned char* scratch,
                                    int lane) {
    using T = Ty<DT>;
    if constexpr (!ORN) {
        unsigned x0 = T::pack(acc0[0], acc0[1]), x1 = T::pack(acc0[2], acc0[3]);
        unsigned y0 = T::pack(acc1[0], acc1[1]), y1 = T::pack(acc1[2], acc1[3]);
        if constexpr (MODE == MODE_RELABEL) {
            return u4_t{x0, x1, y0, y1};
        } else if constexpr (MODE == MODE_PERMLANE) {
            regroup_pairs(x0, x1, y0, y1);
            return u4_t{x0, x1, y0, y1};
        } else if constexpr (MODE == MODE_BPERM) {
            return exchange32<4>(u4_t{x0, x1, y0, y1}, code.lo);
        } else {
            const int m = lane & 15, g = lane >> 4;
            unsigned char* row = scratch + m * LdsRemap<DT>::PITCH;
            *(u2_t*)(row + (4 * g) * 2) = u2_t{x0, x1};
            *(u2_t*)(row + (16 + 4 * g) * 2) = u2_t{y0, y1};
            wave_lds_fence();
            u4_t v = *(const u4_t*)(row + 16 * g);
            wave_lds_fence();
            return v;
        }
    } else {
        // plain orientation: every element changes lane; move single 16-bit values
        static_assert(MODE == MODE_BPERM || MODE == MODE_LDS, "orientation N needs BPERM or LDS");
        code_t h;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            h[v] = T::pack(acc0[v], 0.0f) & 0xFFFFu;
            h[4 + v] = T::pack(acc1[v], 0.0f) & 0xFFFFu;
        }
        if constexpr (MODE == MODE_BPERM) {
            const code_t dst = exchange32<8>(h, code);
            return u4_t{dst[0] | (dst[1] << 16), dst[2] | (dst[3] << 16), dst[4] | (dst[5] << 16),
                        dst[6] | (dst[7] << 16)};
        } else {
            const int n = lane & 15, g = lane >> 4;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                unsigned char* r = scratch + (4 * g + v) * LdsRemap<DT>::PITCH;
                *(unsigned short*)(r + n * 2) = (unsigned short)h[v];
                *(unsigned short*)(r + (16 + n) * 2) = (unsigned short)h[4 + v];
            }
            wave_lds_fence();
            u4_t v = *(const u4_t*)(scratch + n * LdsRemap<DT>::PITCH + 16 * g);
            wave_lds_fence();
            return v;
        }
    }
}

// fp64 rearrangement of one accumulator tile -> four K-steps of 4.
// The fp64 accumulator interleaves rows: register v of lane group g holds row
// g + 4v of the tile.  Orientation T (tile = C0^T): lane (m = l%16, g) holds
// row m of C0, columns g + 4v -- which is already what K-step v of the next
// GEMM wants from lane group g (k = 4v + g).  The rules agree and the operator
// fuses directly; RELABEL and PERMLANE pass the registers through, BPERM runs
// the (identity) coordination rounds, LDS goes through memory.
// Orientation N (tile = C0): lane holds column l%16, rows g + 4v; every
// element changes lane.
template <int MODE, bool ORN>
__device__ inline void remap_unit64(d4_t acc, double (&out)[4], code_t code, unsigned char* scratch,
                                    int lane) {
    double r[4] = {acc[0], acc[1], acc[2], acc[3]};
    constexpr int P = LdsRemap<DT_F64>::PITCH;
    if constexpr (!ORN) {
        if constexpr (MODE == MODE_RELABEL || MODE == MODE_PERMLANE) {
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = r[i];
        } else if constexpr (MODE == MODE_BPERM) {
            exchange64(r, out, code.lo);
        } else {
            const int m = lane & 15, g = lane >> 4;
            unsigned char* row = scratch + m * P;
#pragma unroll
            for (int v = 0; v < 4; ++v) *(double*)(row + (g + 4 * v) * 8) = r[v];
            wave_lds_fence();
#pragma unroll
            for (int s = 0; s < 4; ++s) out[s] = *(const double*)(row + (4 * s + g) * 8);
            wave_lds_fence();
        }
    } else {
        static_assert(MODE == MODE_BPERM || MODE == MODE_LDS, "orientation N needs BPERM or LDS");
        if constexpr (MODE == MODE_BPERM) {
            exchange64(r, out, code.lo);
        } else {
            const int n = lane & 15, g = lane >> 4;
#pragma unroll
            for (int v = 0; v < 4; ++v) *(double*)(scratch + (g + 4 * v) * P + n * 8) = r[v];
            wave_lds_fence();
#pragma unroll
            for (int s = 0; s < 4; ++s) out[s] = *(const double*)(scratch + n * P + (4 * s + g) * 8);
            wave_lds_fence();
        }
    }
}

// ---------------------------------------------------------------------------
// Weights in LDS, fragment-major: the operand fragment (tile t, K-step ks)
// occupies 64 lanes x FB bytes; lane l = n%16 + 16*g holds B[k(ks,g,u)][16t+n%16]
// for its slots u.
// ---------------------------------------------------------------------------
// fp64 K order: K-step and lane group of row k (one slot per lane and K-step).
template <int KM>
__device__ inline void kmap64(int k, int* ks, int* g) {
    if constexpr (KM == KM_PAIR64) {
        const int j = k >> 3, r = k & 7;
        *g = r >> 1;
        *ks = 2 * j + (r & 1);
    } else if constexpr (KM == KM_REL) {
        // the fp64 accumulator's order: K-step 4j + v, lane group g holds
        // k = 16j + g + 4v -- the same as the natural order
        const int j = k >> 4, r = k & 15;
        *g = r & 3;
        *ks = 4 * j + (r >> 2);
    } else {
        *ks = k >> 2;
        *g = k & 3;
    }
}

// fp64 weights: one matrix (KD x ND, row-major in global memory) -> LDS, cut
// into units of 2 columns of one row (one 16-byte load, two 8-byte slots).
// Unit u of the matrix is handled by thread u mod NTHREADS.
template <int DT, int KD, int ND, int KM, int NTHREADS>
struct WStage {
    static_assert(DT == DT_F64, "16-bit weights are staged by stage_tr16");
    static constexpr int KS = KD / Ty<DT>::KW;
    static constexpr int UN = ND / 2;                           // units per row
    static constexpr int UNITS = KD * UN;
    static constexpr int ITERS = (UNITS + NTHREADS - 1) / NTHREADS;
    static constexpr int VGPRS = ITERS * 4;                     // to hold all of a thread's units
    typedef u4_t unit_t[1];

    __device__ static inline void load(unit_t& r, const void* Bg, int64_t ldb, int u) {
        const double* B = (const double*)Bg;
        r[0] = *(const u4_t*)(B + (int64_t)(u / UN) * ldb + (u % UN) * 2);
    }
    __device__ static inline void store(unsigned char* lds, const unit_t& r, int u) {
        const int k = u / UN, n0 = (u % UN) * 2;
        int ks, g;
        kmap64<KM>(k, &ks, &g);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int n = n0 + c, t = n >> 4, lane = (n & 15) + 16 * g;
            *(u2_t*)(lds + ((t * KS + ks) * 64 + lane) * 8) = u2_t{r[0][2 * c], r[0][2 * c + 1]};
        }
    }
};

// Stage one matrix in batches: the loads of a batch of units are all issued
// before any of them is written.
template <int DT, int KD, int ND, int KM, int NTHREADS>
__device__ inline void stage_weights(unsigned char* lds, const void* Bg, int64_t ldb, int tid) {
    using W = WStage<DT, KD, ND, KM, NTHREADS>;
    constexpr int BATCH = W::ITERS < 2 ? W::ITERS : 2;
    for (int i0 = 0; i0 < W::ITERS; i0 += BATCH) {
        typename W::unit_t r[BATCH];
#pragma unroll
        for (int q = 0; q < BATCH; ++q) {
            const int u = tid + (i0 + q) * NTHREADS;
            if (u < W::UNITS) W::load(r[q], Bg, ldb, u);
        }
#pragma unroll
        for (int q = 0; q < BATCH; ++q) {
            const int u = tid + (i0 + q) * NTHREADS;
            if (u < W::UNITS) W::store(lds, r[q], u);
        }
    }
}

// ---------------------------------------------------------------------------
// Compile-time configuration of one kernel instance.
// ---------------------------------------------------------------------------
template <int DT_, int NST_, int D0, int D1, int D2, int D3, int MODE_, bool ORN_, int MT_,
          int WAVES_, int KM0_ = (DT_ == DT_F64 ? KM_PAIR64 : KM_NAT), int PF_ = 2, int FW_ = 3>
struct Cfg {
    static constexpr int DT = DT_, NST = NST_, MODE = MODE_, MT = MT_, WAVES = WAVES_;
    static constexpr int PF = PF_;   // A tiles loaded ahead of the one being computed
    static constexpr int FW = FW_;   // weight fragments in flight from LDS
    static constexpr bool ORN = ORN_;
    static constexpr int KM0 = KM0_;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int ROWS_WAVE = 16 * MT, ROWS_WG = ROWS_WAVE * WAVES;
    static constexpr int dim(int i) { return i == 0 ? D0 : i == 1 ? D1 : i == 2 ? D2 : D3; }
    static constexpr int KW = Ty<DT>::KW, FB = Ty<DT>::FB, ELT = Ty<DT>::ELT;
    static constexpr int KS(int s) { return dim(s) / KW; }
    static constexpr int NT(int s) { return dim(s + 1) / 16; }
    static constexpr int NF(int s) { return s < NST ? NT(s) * KS(s) : 1; }   // fragments per stage
    static constexpr int wbytes(int s) { return s < NST ? NT(s) * KS(s) * 64 * FB : 0; }
    static constexpr int woff(int s) { return s == 0 ? 0 : woff(s - 1) + wbytes(s - 1); }
    static constexpr int WBYTES = woff(3) + 0;
    // per-wave LDS region: the D staging tile, shared with the LDS rearrangement
    static constexpr int NLAST_ = (NST == 1 ? D1 : NST == 2 ? D2 : D3);
    static constexpr int DSTAGE = 16 * MT * NLAST_ * Ty<DT>::ELT;
    static constexpr int WSCRATCH = (MODE == MODE_LDS && NST > 1 && LdsRemap<DT>::BYTES > DSTAGE)
                                        ? LdsRemap<DT>::BYTES : DSTAGE;
    static constexpr int SCRATCH = WAVES * WSCRATCH;
    // 16-bit weights are staged row-major through the area after the weight
    // slots before the first tile: widen it to hold all of them at once where
    // LDS allows (their row-major size equals their fragment-major size)
    static constexpr int STAGE = (DT != DT_F64 && WBYTES > SCRATCH && 2 * WBYTES <= 160 * 1024)
                                     ? WBYTES : SCRATCH;
    static constexpr int LDS_BYTES = WBYTES + STAGE;
    static constexpr int KMS(int s) { return s == 0 ? KM0 : (MODE == MODE_RELABEL ? KM_REL : KM_NAT); }
    static constexpr int NLAST = dim(NST);
    // memory operations of the A prefetch prologue (16-bit): per tile MT x KS(0)
    // 16-byte loads and one flush of dummy D stores (16-byte, whole rows)
    static constexpr int PROLOGUE_OPS = PF * (MT * (D0 / 32) + 16 * MT * NLAST_ * ELT / 16 / 64);
    static_assert(LDS_BYTES <= 160 * 1024, "weights do not fit in LDS");
    static_assert(DT == DT_F64 || D0 % 32 == 0, "K must be a multiple of 32");
    static_assert(DT == DT_F64 || NST < 2 || (D1 % 32 == 0 && (NST < 3 || D2 % 32 == 0)),
                  "intermediate widths must be multiples of 32");
    static_assert(DT != DT_F64 || D0 % 8 == 0, "fp64 K must be a multiple of 8");
};

// A operand tile of one wave: MT sub-tiles of 16 rows, all K-steps.
template <class C>
__device__ inline void load_a(typename Ty<C::DT>::op_t (&a)[C::MT][C::KS(0)],
                              __amdgpu_buffer_rsrc_t rs, int64_t lda, int lane) {
    const int m = lane & 15, g = lane >> 4;
    if constexpr (C::DT != DT_F64) {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < C::KS(0); ++ks)
                a[mt][ks] = ld128(rs, (uint32_t)(((16 * mt + m) * lda + 32 * ks + 8 * g) * 2));
    } else if constexpr (C::KM0 == KM_PAIR64) {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int j = 0; j < C::dim(0) / 8; ++j) {
                const u4_t v = ld128(rs, (uint32_t)(((16 * mt + m) * lda + 8 * j + 2 * g) * 8));
                a[mt][2 * j] = djoin(u2_t{v[0], v[1]});
                a[mt][2 * j + 1] = djoin(u2_t{v[2], v[3]});
            }
    } else {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int ks = 0; ks < C::KS(0); ++ks)
                a[mt][ks] = djoin(ld64(rs, (uint32_t)(((16 * mt + m) * lda + 4 * ks + g) * 8)));
    }
}

// One GEMM stage on MFMA: acc[mt][t] = sum_ks W_s(t, ks) (x) op[mt][ks].
// Weight fragments come from LDS, read a window of FW fragments ahead of the
// MFMAs that use them, so LDS latency overlaps the matrix pipe.  Each fragment
// feeds MT MFMAs (one per 16-row sub-tile).
// Output tiles are finished in order and handed, a group at a time, to
// sink(first_tile, group): a group is one K-step of the next stage (two
// 16-column tiles for 16-bit types, one for fp64) or the last, partial group.
// Only one group of accumulators is live at a time, which leaves the
// registers to the A tiles in flight.
template <class C> struct Grp { static constexpr int G = C::DT == DT_F64 ? 1 : 2; };

template <class C, int S, bool ORN_STAGE, class Sink>
__device__ inline void gemm_stage(const unsigned char* lds,
                                  const typename Ty<C::DT>::op_t (&op)[C::MT][C::KS(S)], int lane,
                                  Sink&& sink) {
    using T = Ty<C::DT>;
    using op_t = typename T::op_t;
    using acc_t = typename T::acc_t;
    constexpr int KS = C::KS(S), NT = C::NT(S), NF = NT * KS, FW = C::FW;
    constexpr int G = Grp<C>::G;
    const unsigned char* w = lds + C::woff(S) + lane * C::FB;
    auto frag = [&](int i) { return *(const op_t*)(w + i * 64 * C::FB); };
    acc_t acc[C::MT][G];
    op_t fr[FW];
#pragma unroll
    for (int i = 0; i < FW - 1; ++i)
        if (i < NF) fr[i] = frag(i);
#pragma unroll
    for (int i = 0; i < NF; ++i) {
        if constexpr (FW > 1) {
            if (i + FW - 1 < NF) fr[(i + FW - 1) % FW] = frag(i + FW - 1);
        } else {
            fr[0] = frag(i);
        }
        const int t = i / KS, ks = i % KS;
        if (ks == 0) {
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt) acc[mt][t % G] = acc_t{};
        }
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
            if constexpr (ORN_STAGE)
                acc[mt][t % G] = T::mma(op[mt][ks], fr[i % FW], acc[mt][t % G]);   // C0 = A . B0
            else
                acc[mt][t % G] = T::mma(fr[i % FW], op[mt][ks], acc[mt][t % G]);   // C^T = W^T . X^T
        }
        if (ks == KS - 1 && (t % G == G - 1 || t == NT - 1)) sink(t - t % G, acc);
    }
}

// One finished group of a stage -> operands of the next stage (round, then
// rearrange): K-step t/2 (16-bit) or K-steps 4t..4t+3 (fp64).
template <class C, bool ORN_STAGE, int KSN>
__device__ inline void group_to_operands(int t, const typename Ty<C::DT>::acc_t (&g)[C::MT][Grp<C>::G],
                                         typename Ty<C::DT>::op_t (&op)[C::MT][KSN], code_t code,
                                         unsigned char* scratch, int lane) {
    if constexpr (C::DT != DT_F64) {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
            op[mt][t / 2] = remap_unit16<C::DT, C::MODE, ORN_STAGE>(g[mt][0], g[mt][1], code, scratch, lane);
    } else {
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
            double o[4];
            remap_unit64<C::MODE, ORN_STAGE>(g[mt][0], o, code, scratch, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) op[mt][4 * t + i] = o[i];
        }
    }
}

// Final stage output -> D (rounded).  The accumulator layout spreads a row of
// D over four lane groups (16 rows per store instruction, 64 bytes of each),
// which the memory system handles poorly; the wave therefore writes its tile
// into its private LDS region (16-byte chunks, XOR-swizzled by row to avoid
// bank conflicts), group by group as the tiles finish, and then reads it back
// so that consecutive lanes store consecutive 16-byte chunks of whole rows.
template <class C>
struct DStage {
    static constexpr int RB = C::NLAST * C::ELT;            // bytes per row of D
    static constexpr int CPR = RB / 16;                      // 16-byte chunks per row
    static constexpr int SWZ = (CPR < 16 ? CPR : 16) - 1;    // swizzle mask
    static constexpr int BYTES = C::ROWS_WAVE * RB;
    static_assert(RB % 16 == 0 && (64 % CPR == 0 || CPR % 64 == 0), "row width not supported");
    __device__ static inline int pos(int row, int chunk) {
        return row * RB + ((chunk ^ (row & SWZ)) << 4);
    }
};

template <class C, int S>
__device__ inline void group_to_dstage(int t, const typename Ty<C::DT>::acc_t (&g)[C::MT][Grp<C>::G],
                                       unsigned char* scratch, int lane) {
    using DS = DStage<C>;
    const int m = lane & 15, grp = lane >> 4;
    if constexpr (C::DT != DT_F64) {
        using T = Ty<C::DT>;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
            const int row = 16 * mt + m;
            if (t + 1 < C::NT(S)) {
                const f4_t a0 = g[mt][0], a1 = g[mt][1];
                unsigned x0 = T::pack(a0[0], a0[1]), x1 = T::pack(a0[2], a0[3]);
                unsigned y0 = T::pack(a1[0], a1[1]), y1 = T::pack(a1[2], a1[3]);
                regroup_pairs(x0, x1, y0, y1);          // lane group grp: columns 16t + 8grp ..+7
                *(u4_t*)(scratch + DS::pos(row, 2 * t + grp)) = u4_t{x0, x1, y0, y1};
            } else {                                    // odd last tile: columns 16t + 4grp ..+3
                const f4_t a0 = g[mt][0];
                *(u2_t*)(scratch + DS::pos(row, 2 * t + (grp >> 1)) + (grp & 1) * 8) =
                    u2_t{T::pack(a0[0], a0[1]), T::pack(a0[2], a0[3])};
            }
        }
    } else {
        // lane group grp holds columns grp + 4v; regroup to 4grp + v (32 contiguous bytes)
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt) {
            double a[4] = {g[mt][0][0], g[mt][0][1], g[mt][0][2], g[mt][0][3]};
            transpose_rows64(a);
            const int row = 16 * mt + m;
            const u2_t p0 = dsplit(a[0]), p1 = dsplit(a[1]), p2 = dsplit(a[2]), p3 = dsplit(a[3]);
            *(u4_t*)(scratch + DS::pos(row, 8 * t + 2 * grp)) = u4_t{p0[0], p0[1], p1[0], p1[1]};
            *(u4_t*)(scratch + DS::pos(row, 8 * t + 2 * grp + 1)) = u4_t{p2[0], p2[1], p3[0], p3[1]};
        }
    }
}

// The staged tile -> whole-row, non-temporal 16-byte stores.
template <class C>
__device__ inline void flush_d(__amdgpu_buffer_rsrc_t rs, int64_t ldd, int lane, unsigned char* scratch) {
    using DS = DStage<C>;
    wave_lds_fence();
    constexpr int CHUNKS = C::ROWS_WAVE * DS::CPR;
    static_assert(CHUNKS % 64 == 0, "tile must be whole store instructions");
#pragma unroll
    for (int i = 0; i < CHUNKS / 64; ++i) {
        const int idx = i * 64 + lane, row = idx / DS::CPR, q = idx % DS::CPR;
        const u4_t v = *(const u4_t*)(scratch + DS::pos(row, q));
        st128(rs, (uint32_t)(row * ldd * C::ELT + q * 16), v);
    }
    wave_lds_fence();
}

// 16-bit weights -> fragment-major LDS, by way of the wave-scratch area (free
// before the first tile): rounds of RCH rows of B_s are copied row-major into
// the scratch area (buffer loads that write LDS, 16-byte chunks swizzled by
// row), then each wave turns whole fragments into their slots with two
// transposing reads (ds_read_b64_tr_b16: every 16-lane group gets a 4 x 16
// block back one column per lane) and one contiguous 16-byte write per lane.
// Loads, reads and writes are all conflict-free; nothing is scattered.
constexpr bool kWeightRotation = true;

template <class C>
struct Tr16 {
    // swizzle of row r's 16-byte chunks (CPR per row) such that the 16 rows
    // one transposing read touches (8g + j, or 4g + j for the relabelled
    // order, plus 0 or 4/16) spread their 32-byte pieces over all banks
    template <int CPR>
    __device__ static inline int swz(int r) {
        if constexpr (CPR >= 32) return 2 * ((r & 3) | (((r >> 3) & 3) << 2));
        else if constexpr (CPR == 16) return 2 * ((r & 3) | (((r >> 3) & 1) << 2));
        else return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
    }
    // row (within a 32-row K-step) of slot element u of lane group g
    template <int KM>
    __device__ static inline int krow(int g, int u) {
        if constexpr (KM == KM_REL) return 4 * g + 16 * (u >> 2) + (u & 3);
        else return 8 * g + u;
    }
};

template <class C, int S>
struct Tr16Geom {
    static constexpr int KD = C::dim(S), ND = C::dim(S + 1), KM = C::KMS(S);
    static constexpr int PITCH = ND * 2, CPR = PITCH / 16, RPP = 1024 / PITCH;   // rows per 1 KB piece
    static constexpr int RCH0 = (C::STAGE / PITCH) / 32 * 32;
    static constexpr int RCH = RCH0 < KD ? RCH0 : KD;                            // rows per round
    static constexpr int KS = KD / 32, NT = ND / 16, BYTES = KD * PITCH;
    static_assert(ND % 16 == 0 && 1024 % PITCH == 0 && CPR >= 8 && RCH >= 32 && KD % 32 == 0,
                  "16-bit weight staging");
};

// rows [r0, r0 + rows) of B_S -> scratch area at byte offset off (row-major,
// swizzled), in 1 KB pieces.  Workgroups of one XCD that share these weights
// ask one L2 for them at the same moment; each starts at a different piece
// (rotation by blockIdx / 8), which lets the L2 serve them several times
// faster than when every workgroup asks for the same lines in the same order.
template <class C, int S>
__device__ inline void tr16_copy(unsigned char* scr, int off, const KArgs& args, int b, int r0, int rows,
                                 int wave, int lane) {
    using G = Tr16Geom<C, S>;
    const auto rs = make_rsrc((const char*)args.B[S] + (int64_t)b * args.sB[S] * C::ELT,
                              (uint32_t)(G::KD * args.ldb[S] * C::ELT));
    const int np = rows / G::RPP, rot = kWeightRotation ? (int)(blockIdx.x / 8) % np : 0;
    for (int i = wave; i < np; i += C::WAVES) {
        const int p = i + rot < np ? i + rot : i + rot - np;
        const int r = p * G::RPP + lane / G::CPR, pos = lane % G::CPR;
        lds_dma16<false>(rs, scr + off + p * 1024,
                         (int)((r0 + r) * args.ldb[S] * C::ELT) +
                             ((pos ^ Tr16<C>::template swz<G::CPR>(r)) << 4));
    }
}

// the fragments of those rows (whole K-steps) -> their slots in the weight area
template <class C, int S>
__device__ inline void tr16_slots(unsigned char* lds, const unsigned char* scr, int off, int r0, int rows,
                                  int wave, int lane) {
    using G = Tr16Geom<C, S>;
    using TR = Tr16<C>;
    const int g = lane >> 4, j = (lane >> 2) & 3, q = lane & 3, kst = rows / 32;
    for (int f = wave; f < G::NT * kst; f += C::WAVES) {
        const int t = f / kst, ksl = f % kst;
        const int chunk = 2 * t + (q >> 1);           // 16-byte chunk holding columns 16t + 4q ..
        u4_t out;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r = 32 * ksl + TR::template krow<G::KM>(g, 4 * h + j);
            auto* a = (__attribute__((address_space(3))) unsigned char*)(lds_ptr_t)scr + off + r * G::PITCH +
                      ((chunk ^ TR::template swz<G::CPR>(r)) << 4) + (q & 1) * 8;
            const tr4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr4_t*)a);
            out[2 * h] = ((unsigned)(unsigned short)v[0]) | ((unsigned)(unsigned short)v[1] << 16);
            out[2 * h + 1] = ((unsigned)(unsigned short)v[2]) | ((unsigned)(unsigned short)v[3] << 16);
        }
        *(u4_t*)(lds + C::woff(S) + ((t * G::KS + r0 / 32 + ksl) * 64 + lane) * 16) = out;
    }
}

// All stages' weights.  `issue_a` issues the A prefetch (NA_OPS memory
// operations); it goes out right after the first copies, so its latency
// overlaps the staging, and the waits for the copies leave it in flight.
template <class C, int NA_OPS, class F>
__device__ inline void stage_tr16_all(unsigned char* lds, const KArgs& args, int b, int wave, int lane,
                                      F&& issue_a) {
    using G0 = Tr16Geom<C, 0>;
    using G1 = Tr16Geom<C, (C::NST > 1 ? 1 : 0)>;
    using G2 = Tr16Geom<C, (C::NST > 2 ? 2 : 0)>;
    unsigned char* scr = lds + C::WBYTES;
    constexpr int TOTAL = G0::BYTES + (C::NST > 1 ? G1::BYTES : 0) + (C::NST > 2 ? G2::BYTES : 0);
    if constexpr (TOTAL <= C::STAGE) {
        // everything at once: one wait, one pass
        tr16_copy<C, 0>(scr, 0, args, b, 0, G0::KD, wave, lane);
        if constexpr (C::NST > 1) tr16_copy<C, 1>(scr, G0::BYTES, args, b, 0, G1::KD, wave, lane);
        if constexpr (C::NST > 2) tr16_copy<C, 2>(scr, G0::BYTES + G1::BYTES, args, b, 0, G2::KD, wave, lane);
        issue_a();
        barrier_vm<NA_OPS>();
        tr16_slots<C, 0>(lds, scr, 0, 0, G0::KD, wave, lane);
        if constexpr (C::NST > 1) tr16_slots<C, 1>(lds, scr, G0::BYTES, 0, G1::KD, wave, lane);
        if constexpr (C::NST > 2) tr16_slots<C, 2>(lds, scr, G0::BYTES + G1::BYTES, 0, G2::KD, wave, lane);
        barrier_lds();
    } else {
        // round by round through the scratch area; the A prefetch follows the
        // first round's copies
        bool first = true;
        auto rounds = [&](auto sc) {
            constexpr int S = decltype(sc)::value;
            using G = Tr16Geom<C, S>;
#pragma unroll 1
            for (int r0 = 0; r0 < G::KD; r0 += G::RCH) {
                const int rows = G::KD - r0 < G::RCH ? G::KD - r0 : G::RCH;
                tr16_copy<C, S>(scr, 0, args, b, r0, rows, wave, lane);
                if (first) {
                    issue_a();
                    barrier_vm<NA_OPS>();
                    first = false;
                } else {
                    barrier_vm<0>();
                }
                tr16_slots<C, S>(lds, scr, 0, r0, rows, wave, lane);
                barrier_lds();
            }
        };
        rounds(std::integral_constant<int, 0>{});
        if constexpr (C::NST > 1) rounds(std::integral_constant<int, 1>{});
        if constexpr (C::NST > 2) rounds(std::integral_constant<int, 2>{});
    }
}

template <class C>
__device__ inline void stage_all_weights(unsigned char* lds, const KArgs& args, int b, int tid) {
    stage_weights<C::DT, C::dim(0), C::dim(1), C::KMS(0), C::THREADS>(
        lds + C::woff(0), (const char*)args.B[0] + (int64_t)b * args.sB[0] * C::ELT, args.ldb[0], tid);
    if constexpr (C::NST > 1)
        stage_weights<C::DT, C::dim(1), C::dim(2), C::KMS(1), C::THREADS>(
            lds + C::woff(1), (const char*)args.B[1] + (int64_t)b * args.sB[1] * C::ELT, args.ldb[1], tid);
    if constexpr (C::NST > 2)
        stage_weights<C::DT, C::dim(2), C::dim(3), C::KMS(2), C::THREADS>(
            lds + C::woff(2), (const char*)args.B[2] + (int64_t)b * args.sB[2] * C::ELT, args.ldb[2], tid);
}

// Weights held in registers between their loads and their LDS writes, so the
// A prefetches can be issued in between and the two latencies overlap.  Used
// when every stage's share of a thread fits in a few registers.
template <class C, int S> struct WSt {
    static constexpr bool LIVE = S < C::NST;
    using W = WStage<C::DT, LIVE ? C::dim(S) : 32, LIVE ? C::dim(S + 1) : 16, C::KMS(S), C::THREADS>;
    static constexpr int VGPRS = LIVE ? W::VGPRS : 0;
};
template <class C> struct WHeld {
    static constexpr bool FITS = WSt<C, 0>::VGPRS + WSt<C, 1>::VGPRS + WSt<C, 2>::VGPRS <= 32;
    typename WSt<C, 0>::W::unit_t h0[WSt<C, 0>::W::ITERS];
    typename WSt<C, 1>::W::unit_t h1[WSt<C, 1>::W::ITERS];
    typename WSt<C, 2>::W::unit_t h2[WSt<C, 2>::W::ITERS];

    template <int S, class H>
    __device__ static inline void load1(H& h, const KArgs& args, int b, int tid) {
        if constexpr (WSt<C, S>::LIVE) {
            using W = typename WSt<C, S>::W;
            const char* Bg = (const char*)args.B[S] + (int64_t)b * args.sB[S] * C::ELT;
#pragma unroll
            for (int i = 0; i < W::ITERS; ++i) {
                const int u = tid + i * C::THREADS;
                if (u < W::UNITS) W::load(h[i], Bg, args.ldb[S], u);
            }
        }
    }
    template <int S, class H>
    __device__ static inline void store1(const H& h, unsigned char* lds, int tid) {
        if constexpr (WSt<C, S>::LIVE) {
            using W = typename WSt<C, S>::W;
#pragma unroll
            for (int i = 0; i < W::ITERS; ++i) {
                const int u = tid + i * C::THREADS;
                if (u < W::UNITS) W::store(lds + C::woff(S), h[i], u);
            }
        }
    }
    __device__ inline void load(const KArgs& args, int b, int tid) {
        load1<0>(h0, args, b, tid);
        load1<1>(h1, args, b, tid);
        load1<2>(h2, args, b, tid);
    }
    __device__ inline void store(unsigned char* lds, int tid) const {
        store1<0>(h0, lds, tid);
        store1<1>(h1, lds, tid);
        store1<2>(h2, lds, tid);
    }
};

// ---------------------------------------------------------------------------
// The fused kernel: persistent workgroups over tiles of ROWS_WG rows.
// ---------------------------------------------------------------------------
template <class C>
__device__ __forceinline__ void fused_body(const KArgs& args) {
    using T = Ty<C::DT>;
    using op_t = typename T::op_t;
    using acc_t = typename T::acc_t;
    __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index is uniform across the wave: keep it (and every tile address
    // derived from it) in scalar registers so buffer resources stay uniform
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    unsigned char* scratch = lds + C::WBYTES + wave * C::WSCRATCH;

    code_t code = {}, code2 = {};
    if constexpr (C::MODE == MODE_BPERM && C::NST > 1) {
#pragma unroll
        for (int j = 0; j < kMaxRounds; ++j) {
            code[j] = args.sched[0][j][lane];
            code2[j] = args.sched[1][j][lane];
        }
    }

    // XCD-aware order: block i runs on XCD i % 8; give each XCD a contiguous
    // range of logical workgroups (hence of tiles and batches).
    const int G = gridDim.x, bid = blockIdx.x;
    const int lid = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
    const int per = args.total_tiles / G, extra = args.total_tiles % G;
    const int t0 = lid * per + (lid < extra ? lid : extra);
    const int t1 = t0 + per + (lid < extra ? 1 : 0);
    if (t0 >= t1) return;

    const int TB = args.tiles_per_batch;
    // Tiles past the workgroup's range get an empty resource: their loads
    // return zeros without touching memory.  Issuing them unconditionally
    // keeps the count of loads in flight the same on every path, so the
    // compiler's wait counts let the prefetched tiles stay in flight.
    int t_end = t1;   // end of the current batch segment
    auto a_rsrc = [&](int t) {
        const bool live = t < t_end;
        const int tc = live ? t : t0;
        const int b = tc / TB;
        const int64_t row0 = (int64_t)(tc % TB) * C::ROWS_WG + wave * C::ROWS_WAVE;
        int64_t rows = args.M - row0;
        rows = rows < 0 ? 0 : (rows > C::ROWS_WAVE ? C::ROWS_WAVE : rows);
        if (!live) rows = 0;
        const char* base = (const char*)args.A + ((int64_t)b * args.sA + (rows ? row0 : 0) * args.lda) * C::ELT;
        return make_rsrc(base, (uint32_t)(rows * args.lda * C::ELT));
    };

    auto process = [&](int t, const op_t (&a)[C::MT][C::KS(0)]) {
        const int b = t / TB;
        const int64_t row0 = (int64_t)(t % TB) * C::ROWS_WG + wave * C::ROWS_WAVE;
        int64_t rows = args.M - row0;
        rows = rows < 0 ? 0 : (rows > C::ROWS_WAVE ? C::ROWS_WAVE : rows);
        const auto d_rs = make_rsrc(
            (char*)args.D + ((int64_t)b * args.sD + (rows ? row0 : 0) * args.ldd) * C::ELT,
            (uint32_t)(rows * args.ldd * C::ELT));

        auto to_d = [&](int tg, const acc_t (&g)[C::MT][Grp<C>::G]) {
            group_to_dstage<C, C::NST - 1>(tg, g, scratch, lane);
        };
        if constexpr (C::NST == 1) {
            gemm_stage<C, 0, C::ORN>(lds, a, lane, to_d);
        } else {
            op_t op1[C::MT][C::KS(1)];
            gemm_stage<C, 0, C::ORN>(lds, a, lane, [&](int tg, const acc_t (&g)[C::MT][Grp<C>::G]) {
                group_to_operands<C, C::ORN>(tg, g, op1, code, scratch, lane);
            });
            if constexpr (C::NST == 2) {
                gemm_stage<C, 1, false>(lds, op1, lane, to_d);
            } else {
                op_t op2[C::MT][C::KS(2)];
                gemm_stage<C, 1, false>(lds, op1, lane, [&](int tg, const acc_t (&g)[C::MT][Grp<C>::G]) {
                    group_to_operands<C, false>(tg, g, op2, code2, scratch, lane);
                });
                gemm_stage<C, 2, false>(lds, op2, lane, to_d);
            }
        }
        flush_d<C>(d_rs, args.ldd, lane, scratch);
    };

    const auto no_rsrc = make_rsrc(args.D, 0u);

    // The workgroup's tiles, one batch (one set of weights) at a time.  Within
    // a batch, A tiles stream through a ring of PF+1 register sets; the loop is
    // unrolled by the ring size so every set keeps its registers (no copies,
    // which would wait on loads still in flight) and PF tiles are always being
    // fetched.  Weights are loaded before the segment, so inside it they are
    // loop-invariant in LDS.
    constexpr int RING = C::PF + 1;
    op_t ring[RING][C::MT][C::KS(0)];
    int t = t0;
    while (t < t1) {
        const int b = t / TB;
        t_end = (b + 1) * TB < t1 ? (b + 1) * TB : t1;
        __syncthreads();
        // Prologue: each prefetched tile is followed by one tile's worth of
        // stores to an empty resource (dropped by the hardware), so that on
        // entry to the loop the loads in flight sit behind as many memory
        // operations as in the steady state and the first rounds wait no
        // longer than the later ones.
        auto prologue = [&]() {
#pragma unroll
            for (int i = 0; i < C::PF; ++i) {
                load_a<C>(ring[i], a_rsrc(t + i), args.lda, lane);
                flush_d<C>(no_rsrc, args.ldd, lane, scratch);
            }
        };
        if constexpr (C::DT != DT_F64) {
            stage_tr16_all<C, C::PROLOGUE_OPS>(lds, args, b, wave, lane, prologue);
        } else if constexpr (WHeld<C>::FITS) {
            // weight loads, then the A prefetches, then the weights' LDS
            // writes: the wait for the weights (memory counters are in
            // order) leaves the A loads in flight
            WHeld<C> wh;
            wh.load(args, b, tid);
            prologue();
            wh.store(lds, tid);
        } else {
            // weights first, so that their wait does not include the A loads
            stage_all_weights<C>(lds, args, b, tid);
            prologue();
        }
        __syncthreads();
        // Every phase either runs or leaves the loop, so no path reaches a
        // later phase (or the next round) with fewer loads in flight than the
        // steady state.
        for (;;) {
            bool done = false;
#pragma unroll
            for (int ph = 0; ph < RING; ++ph) {
                if (!done) {
                    load_a<C>(ring[(ph + C::PF) % RING], a_rsrc(t + C::PF), args.lda, lane);
                    process(t, ring[ph]);
                    done = ++t >= t_end;
                }
            }
            if (done) break;
        }
    }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void fused_kernel(KArgs args) {
    fused_body<C>(args);
}


// ---------------------------------------------------------------------------
// Executor of compiled coordination rounds (any relation of 64 x E 32-bit
// elements, E <= 16): in round j every lane offers one of its elements and
// takes one from the lane its code names, into the slot its code names --
// one ds_bpermute per round.  code[j][lane] = p | give << 6 | r << 10.
// ---------------------------------------------------------------------------
constexpr int kExecMax = 16;
struct ExecArgs {
    int32_t elems, rounds;
    uint16_t code[kExecMax][64];
};

template <int MAXE = kExecMax>
__global__ __launch_bounds__(64) void remap_exec_kernel(const uint32_t* in, uint32_t* out, ExecArgs args) {
    const int lane = threadIdx.x, E = args.elems;
    unsigned x[MAXE], y[MAXE];
#pragma unroll
    for (int e = 0; e < MAXE; ++e) {
        x[e] = e < E ? in[lane * E + e] : 0u;
        y[e] = 0u;
    }
    for (int j = 0; j < args.rounds; ++j) {
        const unsigned c = args.code[j][lane];
        const int src = c & 63, give = (c >> 6) & 15, slot = (c >> 10) & 15;
        unsigned v = 0;
#pragma unroll
        for (int e = 0; e < MAXE; ++e) v = e == give ? x[e] : v;   // selects, no indexing
        const unsigned got = (unsigned)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
#pragma unroll
        for (int e = 0; e < MAXE; ++e) y[e] = e == slot ? got : y[e];
    }
#pragma unroll
    for (int e = 0; e < MAXE; ++e)
        if (e < E) out[lane * E + e] = y[e];
}

// ---------------------------------------------------------------------------
// Probe: one remap unit on index payloads, through the same executors.
// in/out: 64 lanes x E elements (uint16 for 16-bit types, uint64 for fp64).
// ---------------------------------------------------------------------------
template <int DT, int MODE, bool ORN>
__global__ __launch_bounds__(64) void remap_probe_kernel(const void* in, void* out, KArgs args) {
    __shared__ __attribute__((aligned(16))) unsigned char scratch[LdsRemap<DT>::BYTES];
    const int lane = threadIdx.x;
    code_t code;
#pragma unroll
    for (int j = 0; j < kMaxRounds; ++j) code[j] = args.sched[0][j][lane];
    if constexpr (DT != DT_F64) {
        const unsigned short* x = (const unsigned short*)in + lane * 8;
        unsigned w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = x[2 * i] | ((unsigned)x[2 * i + 1] << 16);
        u4_t v;
        if constexpr (!ORN) {
            // feed the pre-packed pairs through the same network as the kernel
            unsigned x0 = w[0], x1 = w[1], y0 = w[2], y1 = w[3];
            if constexpr (MODE == MODE_RELABEL) {
                v = u4_t{x0, x1, y0, y1};
            } else if constexpr (MODE == MODE_PERMLANE) {
                regroup_pairs(x0, x1, y0, y1);
                v = u4_t{x0, x1, y0, y1};
            } else if constexpr (MODE == MODE_BPERM) {
                v = exchange32<4>(u4_t{x0, x1, y0, y1}, code.lo);
            } else {
                const int m = lane & 15, g = lane >> 4;
                unsigned char* row = scratch + m * LdsRemap<DT>::PITCH;
                *(u2_t*)(row + (4 * g) * 2) = u2_t{x0, x1};
                *(u2_t*)(row + (16 + 4 * g) * 2) = u2_t{y0, y1};
                wave_lds_fence();
                v = *(const u4_t*)(row + 16 * g);
            }
        } else {
            code_t h;
#pragma unroll
            for (int i = 0; i < 8; ++i) h[i] = x[i];
            if constexpr (MODE == MODE_BPERM) {
                const code_t dst = exchange32<8>(h, code);
                v = u4_t{dst[0] | (dst[1] << 16), dst[2] | (dst[3] << 16), dst[4] | (dst[5] << 16),
                         dst[6] | (dst[7] << 16)};
            } else {
                const int n = lane & 15, g = lane >> 4;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    unsigned char* r = scratch + (4 * g + q) * LdsRemap<DT>::PITCH;
                    *(unsigned short*)(r + n * 2) = (unsigned short)h[q];
                    *(unsigned short*)(r + (16 + n) * 2) = (unsigned short)h[4 + q];
                }
                wave_lds_fence();
                v = *(const u4_t*)(scratch + n * LdsRemap<DT>::PITCH + 16 * g);
            }
        }
        *(u4_t*)((unsigned short*)out + lane * 8) = v;
    } else {
        const double* x = (const double*)in + lane * 4;
        d4_t acc = {x[0], x[1], x[2], x[3]};
        double o[4];
        remap_unit64<MODE, ORN>(acc, o, code, scratch, lane);
        double* y = (double*)out + lane * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = o[i];
    }
}

// ---------------------------------------------------------------------------
// Probe: one MFMA on raw operand registers; writes the accumulator registers
// of every lane (64 x C elements).  Used to confirm the layout catalogue.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(64) void mfma_probe_kernel(const void* a, const void* b, void* c) {
    const int lane = threadIdx.x;
    using T = Ty<DT>;
    if constexpr (DT != DT_F64) {
        const u4_t av = ((const u4_t*)a)[lane], bv = ((const u4_t*)b)[lane];
        ((f4_t*)c)[lane] = T::mma(av, bv, f4_t{0.f, 0.f, 0.f, 0.f});
    } else {
        const double av = ((const double*)a)[lane], bv = ((const double*)b)[lane];
        ((d4_t*)c)[lane] = T::mma(av, bv, d4_t{0.0, 0.0, 0.0, 0.0});
    }
}

}  // namespace b2bk
