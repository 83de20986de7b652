// Fused cascade in tf32, the data type of page 1's worked example, on
// gfx950, which has no tf32 matrix instruction.
//
// A tf32 value t (binary32 with 10 fraction bits) is the exact sum of two
// bfloat16 values: hi, the leading 8 significant bits of t, and lo = t - hi,
// which holds the remaining 3.  A product of two tf32 values is then
//     a b = ah bh + ah bl + al bh + al bl,
// each term an exact product of bfloat16 values, which the bf16 matrix
// instruction forms exactly and sums in fp32.  PASSES = 3 drops al bl (less
// than 2^-14 of |a b|); PASSES = 4 keeps it, so every tf32 product is exact
// and only the order of the fp32 sums differs from a tf32 dot product.
//
// Layouts are those of the 32x32x16 run-time-width kernels: the first GEMM
// is computed transposed so that lane l holds 16 values of row l%32 of the
// result, and the next GEMM takes them in relabelled K order (K-step 2t+s of
// 32-column tile t takes result register 8s+u in slot u, nothing moves).  A
// and B are fp32 in memory; each weight matrix sits in LDS twice, as its hi
// and lo parts (so 4 bytes per element, like fp32), in the 32-column block
// layout the transposing reads expect.  A is read in natural K order (lane
// l: row l%32, k = 16j + 8(l/32) + 0..7 for K-step j, two 16-byte loads),
// rounded and split in registers; the loads of the next tile are issued
// once the split has consumed this one (before the last GEMM of a cascade,
// where the registers allow).  D is fp32, staged per 32-column
// tile through a 4 KB region per wave so that stores write whole 128-byte
// row segments.
#pragma once
#include "kernels_gen.hpp"

namespace b2bk {

// NST_: GEMMs (1 for the unfused path); MAXD_: bound on every width;
// PASSES_: 3 or 4; WAVES_: 8 (two waves per SIMD, up to 256 registers
// each) or 4 (one wave per SIMD with up to 512).  F0_..F3_: widths fixed at
// compile time (K, N1, ...; all zero: read at run time).  With the widths
// known the K-step and tile loops lose their branches and the weight
// fragment addresses become immediates.
template <int NST_, int MAXD_, int PASSES_, int WAVES_ = 8, int F0_ = 0, int F1_ = 0, int F2_ = 0, int F3_ = 0>
struct Tf32Cfg {
    static constexpr int DT = DT_TF32, NST = NST_, MAXD = MAXD_, PASSES = PASSES_;
    static constexpr bool FIXED = F0_ > 0;
    static constexpr int F(int i) { return i == 0 ? F0_ : i == 1 ? F1_ : i == 2 ? F2_ : F3_; }
    static constexpr int MODE = MODE_RELABEL;
    static constexpr int WAVES = WAVES_, THREADS = 64 * WAVES, ROWS_WAVE = 32, ROWS_WG = ROWS_WAVE * WAVES;
    static constexpr int MKS = MAXD / 16, MNT = MAXD / 32;
    static constexpr int LDS_MAX = 160 * 1024;
    static_assert(MAXD % 32 == 0 && NST >= 1 && NST <= kMaxStages, "config");
    static_assert(PASSES == 3 || PASSES == 4, "passes");
    static_assert(WAVES == 4 || WAVES == 8, "waves");
    static_assert(!FIXED || (F(0) % 32 == 0 && F(0) <= MAXD && F(NST) % 32 == 0 && F(NST) <= MAXD &&
                             (NST < 2 || (F(1) % 32 == 0 && F(1) <= MAXD)) &&
                             (NST < 3 || (F(2) % 32 == 0 && F(2) <= MAXD))),
                  "fixed widths: multiples of 32 within the bound");
};

// LDS bytes: every weight matrix as hi and lo parts (2 x 2 bytes per
// element), then 4 KB of D staging for each of up to 8 waves when that still
// fits 160 KB
__host__ __device__ inline int64_t tf32_weight_bytes(const int32_t* d, int nst) {
    int64_t b = 0;
    for (int s = 0; s < nst; ++s) b += (int64_t)d[s] * d[s + 1] * 4;
    return b;
}
__host__ __device__ inline bool tf32_stage_d(const int32_t* d, int nst) {
    return tf32_weight_bytes(d, nst) + 8 * 4096 <= 160 * 1024;
}
__host__ __device__ inline int64_t tf32_lds_bytes(const int32_t* d, int nst) {
    return tf32_weight_bytes(d, nst) + (tf32_stage_d(d, nst) ? 8 * 4096 : 0);
}

// binary32 encoding of a finite value -> tf32 encoding: nearest-even on the
// low 13 bits (a carry moves to the next binade, or to infinity).  A NaN may
// come out as an infinity; the split below turns either into a NaN product.
__device__ __forceinline__ uint32_t tf32_round_bits(uint32_t u) {
    return (u + 0xFFFu + ((u >> 13) & 1u)) & 0xFFFFE000u;
}

// tf32 encoding t -> hi, lo (binary32 encodings with zero low halves, so
// their upper halves are bfloat16 values) with hi + lo = t exactly: hi keeps
// the leading 8 significant bits of t, lo = t - hi the other 3 (same sign,
// below 2^-7 |t|).  An infinite t gives lo = inf - inf = NaN, so every
// emulated product of a non-finite operand is NaN.
__device__ __forceinline__ void tf32_split(uint32_t t, uint32_t& hi, uint32_t& lo) {
    hi = t & 0xFFFF0000u;
    lo = __float_as_uint(__uint_as_float(t) - __uint_as_float(hi));
}

// upper halves of two binary32 encodings -> one packed pair of bfloat16 (x0 low)
__device__ __forceinline__ uint32_t tf32_pack(uint32_t x0, uint32_t x1) {
    return __builtin_amdgcn_perm(x1, x0, 0x07060302u);
}

// 8 binary32 values (two 16-byte pieces) -> the hi and lo bf16 operands of one K-step
__device__ __forceinline__ void tf32_operand(const u4_t& p0, const u4_t& p1, u4_t& oh, u4_t& ol) {
    uint32_t h[8], l[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        tf32_split(tf32_round_bits(p0[i]), h[i], l[i]);
        tf32_split(tf32_round_bits(p1[i]), h[4 + i], l[4 + i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        oh[i] = tf32_pack(h[2 * i], h[2 * i + 1]);
        ol[i] = tf32_pack(l[2 * i], l[2 * i + 1]);
    }
}

__device__ __forceinline__ f16x_t tf32_mma(u4_t a, u4_t b, f16x_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8_t, a), __builtin_bit_cast(bf8_t, b), c,
                                                   0, 0, 0);
}

// weights of batch b -> LDS as hi and lo parts (16-byte loads of 4 values,
// eight in flight per thread; every thread issues the same loads, those past
// the end through an offset beyond the resource)
template <class C>
__device__ inline void tf32_stage_weights(unsigned char* lds, const GenMat (&mh)[C::NST], const GenMat (&ml)[C::NST],
                                          const KArgs& args, int b) {
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        const GenMat& m = mh[s];
        const int lo_off = ml[s].off - m.off;
        const auto rs = make_rsrc((const char*)args.B[s] + (int64_t)b * args.sB[s] * 4,
                                  (uint32_t)(m.rows * args.ldb[s] * 4));
        const int cpr = m.n / 4, total = m.rows * cpr;
        for (int i0 = 0; i0 < total; i0 += 8 * C::THREADS) {
            u4_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 4;
                v[k] = ld128(rs, i < total ? (uint32_t)((r * args.ldb[s] + c) * 4) : 0xFFFFFFF0u);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 4;
                uint32_t h[4], l[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) tf32_split(tf32_round_bits(v[k][e]), h[e], l[e]);
                if (i < total) {
                    unsigned char* p = lds + m.pos(r, c);
                    *(u2_t*)p = u2_t{tf32_pack(h[0], h[1]), tf32_pack(h[2], h[3])};
                    *(u2_t*)(p + lo_off) = u2_t{tf32_pack(l[0], l[1]), tf32_pack(l[2], l[3])};
                }
            }
        }
    }
}

// A of one wave's 32 rows in natural K order: K-step j is a[2j] (k = 16j +
// 8(l/32) + 0..3) and a[2j+1] (+4..7) of row l%32.  Loads past K go through
// the empty resource (zeros, no memory access).
template <class C, int J0 = 0, int J1 = C::MKS>
__device__ __forceinline__ void tf32_load_a(u4_t (&a)[2 * C::MKS], __amdgpu_buffer_rsrc_t rs,
                                            __amdgpu_buffer_rsrc_t none, int64_t lda, int ks, int lane) {
    const int m = lane & 31, h = lane >> 5;
#pragma unroll
    for (int j = J0; j < J1; ++j) {
        const auto src = j < ks ? rs : none;
        const uint32_t off = (uint32_t)((m * lda + 16 * j + 8 * h) * 4);
        a[2 * j] = ld128(src, off);
        a[2 * j + 1] = ld128(src, off + 16);
    }
}

// One GEMM on one wave's 32 rows: operand K-steps xh / xl (ks of them),
// result tiles of 32 columns in pairs (an odd last tile computed twice, the
// copy dropped), each pair handed to sink(t, acc_t, acc_t+1, two).
template <class C, class Sink>
__device__ __forceinline__ void tf32_gemm(const unsigned char* lds, const GenFrag& fh, const GenFrag& fl,
                                          const u4_t (&xh)[C::MKS], const u4_t (&xl)[C::MKS], int ks, int nt,
                                          Sink&& sink) {
    if constexpr (!C::FIXED) {
        ks = uniform_here(ks);
        nt = uniform_here(nt);
    }
#pragma unroll
    for (int t = 0; t < C::MNT; t += 2) {
        if (t < nt) {
            const bool two = t + 1 < nt;
            const int t1 = two ? t + 1 : t;
            // one K-step of both chains; K-step 0 always exists (every
            // width is at least 32) and starts them from zero, with no
            // accumulator to clear
            auto kstep = [&](int j, f16x_t c0, f16x_t c1, f16x_t& o0, f16x_t& o1) __attribute__((always_inline)) {
                const u4_t wh0 = gen_wfrag(lds, fh, t, j), wl0 = gen_wfrag(lds, fl, t, j);
                const u4_t wh1 = gen_wfrag(lds, fh, t1, j), wl1 = gen_wfrag(lds, fl, t1, j);
                // the small terms first
                if constexpr (C::PASSES == 4) {
                    c0 = tf32_mma(wl0, xl[j], c0);
                    c1 = tf32_mma(wl1, xl[j], c1);
                }
                c0 = tf32_mma(wl0, xh[j], c0);
                c1 = tf32_mma(wl1, xh[j], c1);
                c0 = tf32_mma(wh0, xl[j], c0);
                c1 = tf32_mma(wh1, xl[j], c1);
                o0 = tf32_mma(wh0, xh[j], c0);
                o1 = tf32_mma(wh1, xh[j], c1);
            };
            f16x_t acc0, acc1;
            kstep(0, f16x_t{}, f16x_t{}, acc0, acc1);
#pragma unroll
            for (int j = 1; j < C::MKS; ++j)
                if (j < ks) kstep(j, acc0, acc1, acc0, acc1);
            sink(t, acc0, acc1, two);
        }
    }
}

// The same GEMM with the K-steps outermost: every result tile accumulates at
// once, so each operand K-step is dead after its step (a GEMM between two
// others holds its input and output operands otherwise).
template <class C, class Sink>
__device__ __forceinline__ void tf32_gemm_kouter(const unsigned char* lds, const GenFrag& fh, const GenFrag& fl,
                                                 const u4_t (&xh)[C::MKS], const u4_t (&xl)[C::MKS], int ks,
                                                 int nt, Sink&& sink) {
    if constexpr (!C::FIXED) {
        ks = uniform_here(ks);
        nt = uniform_here(nt);
    }
    // K-step 0 always exists: its products start every tile's chain from
    // zero (tiles past nt are never computed and never read)
    f16x_t acc[C::MNT];
#pragma unroll
    for (int j = 0; j < C::MKS; ++j)
        if (j == 0 || j < ks) {
#pragma unroll
            for (int t = 0; t < C::MNT; ++t)
                if (t < nt) {
                    const u4_t wh = gen_wfrag(lds, fh, t, j), wl = gen_wfrag(lds, fl, t, j);
                    f16x_t c = j == 0 ? f16x_t{} : acc[t];
                    if constexpr (C::PASSES == 4) c = tf32_mma(wl, xl[j], c);
                    c = tf32_mma(wl, xh[j], c);
                    c = tf32_mma(wh, xl[j], c);
                    acc[t] = tf32_mma(wh, xh[j], c);
                }
        }
#pragma unroll
    for (int t = 0; t < C::MNT; t += 2)
        if (t < nt) sink(t, acc[t], acc[t + 1 < C::MNT ? t + 1 : t], t + 1 < nt);
}

// Result tile -> two K-steps (2t, 2t+1) of the next GEMM's hi and lo operands, relabelled.
__device__ __forceinline__ void tf32_to_operand(const f16x_t& acc, u4_t& h0, u4_t& l0, u4_t& h1, u4_t& l1) {
    const u4_t r0 = {__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                     __float_as_uint(acc[3])};
    const u4_t r1 = {__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]),
                     __float_as_uint(acc[7])};
    const u4_t r2 = {__float_as_uint(acc[8]), __float_as_uint(acc[9]), __float_as_uint(acc[10]),
                     __float_as_uint(acc[11])};
    const u4_t r3 = {__float_as_uint(acc[12]), __float_as_uint(acc[13]), __float_as_uint(acc[14]),
                     __float_as_uint(acc[15])};
    tf32_operand(r0, r1, h0, l0);
    tf32_operand(r2, r3, h1, l1);
}

// One 32 x 32 fp32 result tile -> D.  Lane (m = l%32, h = l/32) holds
// columns 8a + 4h + 0..3 (registers 4a..4a+3): 16-byte chunk 2a+h of the
// tile's 128-byte row segment.  Through the staging region (chunks
// XOR-swizzled by row) each store writes 8 rows x 128 bytes; without one
// the chunks go straight to memory.
__device__ __forceinline__ void tf32_store_tile(unsigned char* lds, int stg, const f16x_t& acc,
                                                __amdgpu_buffer_rsrc_t rs, int64_t ldd, int n0, int lane_) {
    // the lane index passes through an empty asm statement so that the
    // compiler computes the store offsets here, per tile, instead of keeping
    // every tile's offsets in registers for the whole kernel (at two waves
    // per SIMD the three-GEMM cascade would spill them)
    int lane = lane_;
    asm volatile("" : "+v"(lane));
    const int m = lane & 31, h = lane >> 5;
    u4_t c[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
        c[a] = u4_t{__float_as_uint(acc[4 * a]), __float_as_uint(acc[4 * a + 1]), __float_as_uint(acc[4 * a + 2]),
                    __float_as_uint(acc[4 * a + 3])};
    if (stg < 0) {
#pragma unroll
        for (int a = 0; a < 4; ++a) st128_part(rs, (uint32_t)((m * ldd + n0 + 8 * a + 4 * h) * 4), c[a]);
        return;
    }
    unsigned char* st = lds + stg;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int chunk = 2 * a + h;
        *(u4_t*)(st + m * 128 + ((chunk ^ (m & 7)) << 4)) = c[a];
    }
    // LDS accesses of one wave complete in order; only the compiler must not
    // move the reads above the writes
    asm volatile("" ::: "memory");
    const int ch = lane & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3);
        const u4_t v = *(const u4_t*)(st + r * 128 + ((ch ^ (r & 7)) << 4));
        st128(rs, (uint32_t)((r * ldd + n0 + 4 * ch) * 4), v);
    }
    asm volatile("" ::: "memory");
}

template <class C>
__device__ __forceinline__ void tf32_body(const KArgs& args) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int d[C::NST + 1];
#pragma unroll
    for (int i = 0; i <= C::NST; ++i) d[i] = C::FIXED ? C::F(i) : args.dims[i];
    GenMat mh[C::NST], ml[C::NST];
    int off = 0;
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        mh[s].init(off, d[s], d[s + 1]);
        ml[s].init(off + d[s] * d[s + 1] * 2, d[s], d[s + 1]);
        off += d[s] * d[s + 1] * 4;
    }
    const int ks0 = d[0] / 16, dn = d[C::NST];
    const int stg = tf32_stage_d(d, C::NST) ? off + wave * 4096 : -1;
    GenFrag fh[C::NST], fl[C::NST];
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        fh[s].init(mh[s], s > 0, lane);
        fl[s].init(ml[s], s > 0, lane);
    }

    TileRange<C::ROWS_WG, C::ROWS_WAVE> tr;
    if (!tr.init(args, wave)) return;
    auto a_rsrc = [&](int t) { return tr.a_rsrc(args.A, args.lda, args.sA, 4, t); };
    const auto no_rsrc = make_rsrc(args.A, 0u);

    u4_t a[2 * C::MKS];
    int t = tr.t0;
    while (t < tr.t1) {
        const int b = t / tr.TB;
        tr.segment(t);
        __syncthreads();   // the previous segment's weight reads are over
        tf32_stage_weights<C>(lds, mh, ml, args, b);
        tf32_load_a<C>(a, a_rsrc(t), no_rsrc, args.lda, ks0, lane);
        __syncthreads();
        for (; t < tr.t_end; ++t) {
            u4_t xh[C::MKS], xl[C::MKS];
#pragma unroll
            for (int j = 0; j < C::MKS; ++j) tf32_operand(a[2 * j], a[2 * j + 1], xh[j], xl[j]);
            // this tile's A is consumed: the next one's loads go out -- all
            // at once where the registers allow (a single GEMM, or one wave
            // per SIMD), else in two parts, the second once the split
            // operands of the first GEMM are no longer live.  Run-time
            // widths: a quarter now and the rest before the last GEMM for two
            // GEMMs, all of it before the last GEMM for three (whose middle
            // GEMM holds its input and output operands).  Widths compiled in
            // (fewer registers for addresses and loop state): half now, the
            // rest before the last GEMM, or after the first of three.
            constexpr bool EARLY = C::NST == 1 || C::WAVES == 4;
            constexpr bool MID = C::FIXED && C::NST == 3 && !EARLY;
            constexpr int Q = C::FIXED ? C::MKS / 2 : (EARLY || C::NST < 3) ? C::MKS / 4 : 0;   // K-steps loaded now
            auto issue_next = [&]() __attribute__((always_inline)) {
                tf32_load_a<C, Q, C::MKS>(a, a_rsrc(t + 1), no_rsrc, args.lda, ks0, lane);
            };
            tf32_load_a<C, 0, Q>(a, a_rsrc(t + 1), no_rsrc, args.lda, ks0, lane);
            if constexpr (EARLY) issue_next();

            const auto d_rs = tr.rsrc(args.D, args.ldd, args.sD, 4, t);
            auto to_d = [&](int tt, const f16x_t& a0, const f16x_t& a1, bool two) __attribute__((always_inline)) {
                tf32_store_tile(lds, stg, a0, d_rs, args.ldd, 32 * tt, lane);
                if (two) tf32_store_tile(lds, stg, a1, d_rs, args.ldd, 32 * tt + 32, lane);
            };
            if constexpr (C::NST == 1) {
                tf32_gemm<C>(lds, fh[0], fl[0], xh, xl, ks0, dn / 32, to_d);
            } else {
                // the operands of stage s come from (oAh, oAl) for s odd, (oBh, oBl) for s even
                u4_t oAh[C::MKS], oAl[C::MKS], oBh[C::MKS], oBl[C::MKS];
                auto to_ops = [&](u4_t (&oh)[C::MKS], u4_t (&ol)[C::MKS]) __attribute__((always_inline)) {
                    return [&oh, &ol](int tt, const f16x_t& a0, const f16x_t& a1, bool two)
                               __attribute__((always_inline)) {
                                   tf32_to_operand(a0, oh[2 * tt], ol[2 * tt], oh[2 * tt + 1], ol[2 * tt + 1]);
                                   if (two)
                                       tf32_to_operand(a1, oh[2 * tt + 2], ol[2 * tt + 2], oh[2 * tt + 3],
                                                       ol[2 * tt + 3]);
                               };
                };
                tf32_gemm<C>(lds, fh[0], fl[0], xh, xl, ks0, d[1] / 32, to_ops(oAh, oAl));
                if constexpr (MID) issue_next();
                gen_static_for<1, C::NST - 1>([&](auto sc) __attribute__((always_inline)) {
                    constexpr int S = decltype(sc)::value;
                    if constexpr (S % 2 == 1)
                        tf32_gemm_kouter<C>(lds, fh[S], fl[S], oAh, oAl, d[S] / 16, d[S + 1] / 32, to_ops(oBh, oBl));
                    else
                        tf32_gemm_kouter<C>(lds, fh[S], fl[S], oBh, oBl, d[S] / 16, d[S + 1] / 32, to_ops(oAh, oAl));
                });
                constexpr int L = C::NST - 1;
                if constexpr (!EARLY && !MID) issue_next();
                if constexpr (L % 2 == 1) tf32_gemm<C>(lds, fh[L], fl[L], oAh, oAl, d[L] / 16, dn / 32, to_d);
                else tf32_gemm<C>(lds, fh[L], fl[L], oBh, oBl, d[L] / 16, dn / 32, to_d);
            }
        }
    }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void tf32_kernel(KArgs args) {
    tf32_body<C>(args);
}

}  // namespace b2bk
