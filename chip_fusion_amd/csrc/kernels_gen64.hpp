// Fused cascade in fp64 on v_mfma_f64_16x16x4_f64 with the widths given at
// run time (K a multiple of 8, N1.. multiples of 16, each at most the
// instance's bound).
//
// Layouts (gfx950, confirmed by the one-instruction probe): operand A, lane l
// holds row l%16 and k = l/16; operand B, k = l/16 and column l%16; result,
// lane l holds column l%16 and rows l/16 + 4v (v < 4).  The first GEMM is
// computed transposed, C0^T = B0^T . A^T, so lane l holds the values of row
// l%16 of C0 at columns 16t + l/16 + 4v.  Page 1 ("数据处理方法、装置、设备
// 及介质", detailed description) rearranges the result only where the two
// register layouts differ; here the next GEMM's operand for K-step 4t+v wants
// exactly register v of result tile t in the same lane (k = 16t + 4v + l/16):
// the layouts coincide and nothing moves.  The first GEMM reads A 16 bytes at
// a time, so its K-step 2p+e holds k = 8p + 2*(l/16) + e in every operand.
//
// Weights live in LDS in blocks of 16 columns (all rows x 128 bytes each);
// every weight fragment is one 8-byte read per lane whose address moves by
// immediates in the K-step.  Each wave owns 16 rows of a 128-row tile; output
// tiles go in groups (independent accumulation chains); D leaves through an
// 8 KB staging region per wave as 512-byte row segments, or straight from
// registers when the weights leave no room.
#pragma once
#include "kernels.hpp"

namespace b2bk {

// NST_: GEMMs (1..6); MAXD_: bound on every width; PF_: A tiles fetched ahead;
// GRP_: output tiles computed together.
// TAIL_: any widths and any leading dimensions and batch strides: K is
// padded to a multiple of 8 and every N to a multiple of 16 on chip (weights
// zero-filled in LDS, A's columns past K read as zero, D's columns past N not
// written).
template <int NST_, int MAXD_, int PF_, int GRP_, bool TAIL_ = false>
struct Gen64Cfg {
    static constexpr int DT = DT_F64, NST = NST_, MAXD = MAXD_, PF = PF_, GRP = GRP_;
    static constexpr bool TAIL = TAIL_;
    static constexpr int MODE = MODE_RELABEL;                 // the layouts coincide
    static constexpr int WAVES = 8, THREADS = 64 * WAVES, ROWS_WAVE = 16, ROWS_WG = ROWS_WAVE * WAVES;
    static constexpr int MKS = MAXD / 4, MNT = MAXD / 16;     // K-steps, 16-column tiles
    static constexpr int LDS_MAX = 160 * 1024, STG = 16 * 64 * 8;   // staging bytes per wave
    static_assert(MAXD % 16 == 0 && NST >= 1 && NST <= kMaxStages && (PF == 0 || PF == 1), "config");
    static_assert(GRP == 2 || GRP == 4, "tile group");
};

// the widths a kernel lays out: K to a multiple of 8 and every N to one of
// 16 where the kernel takes tails, else as given
__host__ __device__ inline void gen64_pad(const int32_t* d, int nst, bool tail, int32_t* out) {
    for (int i = 0; i <= nst; ++i) out[i] = !tail ? d[i] : i == 0 ? (d[i] + 7) / 8 * 8 : (d[i] + 15) / 16 * 16;
}

__host__ __device__ inline int64_t gen64_weight_bytes(const int32_t* d, int nst) {
    int64_t b = 0;
    for (int s = 0; s < nst; ++s) b += (int64_t)d[s] * d[s + 1] * 8;
    return b;
}
__host__ __device__ inline bool gen64_stage_d(const int32_t* d, int nst) {
    return gen64_weight_bytes(d, nst) + 8 * (16 * 64 * 8) <= 160 * 1024;
}
__host__ __device__ inline int64_t gen64_lds_bytes(const int32_t* d, int nst) {
    return gen64_weight_bytes(d, nst) + (gen64_stage_d(d, nst) ? 8 * (16 * 64 * 8) : 0);
}

// Per-lane constants of one matrix's weight fragments: fragment (16-column
// tile t, K-step j) of lane (c = l%16, g = l/16) is W[k][16t + c] with
//   first GEMM:  k = 8(j/2) + 2g + j%2     (pairs of K-steps read together)
//   later GEMMs: k = 16(j/4) + 4(j%4) + g  (the previous result's layout)
// at base + t tstride + 128 kj(j), kj(j) = 8(j/2) + j%2 or 16(j/4) + 4(j%4).
struct Gen64Frag {
    int base, tstride;
    __device__ inline void init(int off, int rows, bool first, int lane) {
        const int c = lane & 15, g = lane >> 4;
        base = off + (first ? 2 * g : g) * 128 + c * 8;
        tstride = rows * 128;
    }
};

template <bool FIRST>
__device__ __forceinline__ double gen64_wfrag(const unsigned char* lds, const Gen64Frag& fr, int t, int j) {
    const int kj = FIRST ? 8 * (j / 2) + (j % 2) : 16 * (j / 4) + 4 * (j % 4);
    return *(const double*)(lds + fr.base + t * fr.tstride + 128 * kj);
}

// The same copy by buffer loads that write LDS: one instruction moves 8 rows
// x 128 bytes of one 16-column block -- lane l takes 16-byte piece l%8 of row
// 8i + l/8 -- which is 1 KB of contiguous LDS.  Widths are whole blocks here
// (the tail kernels stage through registers).
template <class C>
__device__ inline void gen64_copy_weights(unsigned char* lds, const int (&d)[C::NST + 1], const KArgs& args, int b,
                                          int wave) {
    const int lane = lane_here();
    int off = 0;
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        const int rows = d[s], n = d[s + 1];
        const auto rs = make_rsrc((const char*)args.B[s] + (int64_t)b * args.sB[s] * 8,
                                  (uint32_t)(rows * args.ldb[s] * 8));
        const int rg = rows / 8, nq = rg * (n / 16);
        for (int q = wave; q < nq; q += C::THREADS / 64) {
            const int blk = q / rg, i = q % rg, r = 8 * i + (lane >> 3);
            lds_dma16<false>(rs, lds + off + blk * rows * 128 + 1024 * i,
                             (int)((r * args.ldb[s] + 16 * blk + 2 * (lane & 7)) * 8));
        }
        off += rows * n * 8;
    }
}

// weights of batch b -> LDS, 16 columns per block (16-byte loads, eight in
// flight per thread, every thread issuing the same loads)
template <class C>
__device__ inline void gen64_stage_weights(unsigned char* lds, const int (&d)[C::NST + 1], const KArgs& args,
                                           int b) {
    int off = 0;
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        const int rows = d[s], n = d[s + 1], cpr = n / 2, total = rows * cpr;   // 16-byte pieces
        const auto rs = make_rsrc((const char*)args.B[s] + (int64_t)b * args.sB[s] * 8,
                                  (uint32_t)(rows * args.ldb[s] * 8));
        for (int i0 = 0; i0 < total; i0 += 8 * C::THREADS) {
            u4_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 2;
                v[k] = ld128(rs, i < total ? (uint32_t)((r * args.ldb[s] + c) * 8) : 0xFFFFFFF0u);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 2;
                if (i < total) *(u4_t*)(lds + off + (c >> 4) * rows * 128 + r * 128 + (c & 15) * 8) = v[k];
            }
        }
        off += rows * n * 8;
    }
}

// A 16-byte piece of two fp64 elements of which `valid` lie inside the row:
// whole, one 16-byte access at any 8-byte alignment; half, one 8-byte
// access; none, nothing (zeros)
__device__ __forceinline__ u4_t ld_pair64(__amdgpu_buffer_rsrc_t rs, uint32_t off, int valid) {
    if (valid >= 2) return ld128(rs, off);
    if (valid == 1) {
        const u2_t x = ld64(rs, off);
        return u4_t{x[0], x[1], 0u, 0u};
    }
    return u4_t{0u, 0u, 0u, 0u};
}
__device__ __forceinline__ void st_pair64(__amdgpu_buffer_rsrc_t rs, uint32_t off, u4_t v, int valid, bool part) {
    if (valid >= 2 && part) st128_part(rs, off, v);
    else if (valid >= 2) st128(rs, off, v);
    else if (valid == 1) __builtin_amdgcn_raw_buffer_store_b64(u2_t{v[0], v[1]}, rs, (int)off, 0, 0);
}

// weights of batch b -> LDS, zero-padded to the laid-out widths d (dt: true)
template <class C>
__device__ inline void gen64_stage_weights_tail(unsigned char* lds, const int (&d)[C::NST + 1],
                                                const int (&dt)[C::NST + 1], const KArgs& args, int b) {
    int off = 0;
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        const int rows = d[s], n = d[s + 1], cpr = n / 2, total = rows * cpr;   // 16-byte pieces
        const int rows_t = dt[s], cols_t = dt[s + 1];
        const auto rs = make_rsrc((const char*)args.B[s] + (int64_t)b * args.sB[s] * 8,
                                  (uint32_t)(rows_t * args.ldb[s] * 8));
        for (int i0 = 0; i0 < total; i0 += 8 * C::THREADS) {
            u4_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 2;
                const int valid = (i < total && r < rows_t) ? cols_t - c : 0;
                v[k] = ld_pair64(rs, (uint32_t)((r * args.ldb[s] + c) * 8), valid);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 2;
                if (i < total) *(u4_t*)(lds + off + (c >> 4) * rows * 128 + r * 128 + (c & 15) * 8) = v[k];
            }
        }
        off += rows * n * 8;
    }
}

// gen64_load_a with a K tail (K: the true width)
template <class C>
__device__ __forceinline__ void gen64_load_a_tail(double (&a)[C::MKS], __amdgpu_buffer_rsrc_t rs, int64_t lda, int ks,
                                                  int K, int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int p = 0; p < C::MKS / 2; ++p) {
        const int c0 = 8 * p + 2 * g;
        const u4_t v = ld_pair64(rs, (uint32_t)((m * lda + c0) * 8), 2 * p < ks ? K - c0 : 0);
        a[2 * p] = djoin(u2_t{v[0], v[1]});
        a[2 * p + 1] = djoin(u2_t{v[2], v[3]});
    }
}

// A of one wave's 16 rows: load p brings k = 8p + 2g, 8p + 2g + 1 of row l%16,
// the operands of K-steps 2p and 2p+1 (past K: an empty resource, zeros)
template <class C>
__device__ __forceinline__ void gen64_load_a(double (&a)[C::MKS], __amdgpu_buffer_rsrc_t rs,
                                             __amdgpu_buffer_rsrc_t none, int64_t lda, int ks, int lane) {
    const int m = lane & 15, g = lane >> 4;
#pragma unroll
    for (int p = 0; p < C::MKS / 2; ++p) {
        const u4_t v = ld128(2 * p < ks ? rs : none, (uint32_t)((m * lda + 8 * p + 2 * g) * 8));
        a[2 * p] = djoin(u2_t{v[0], v[1]});
        a[2 * p + 1] = djoin(u2_t{v[2], v[3]});
    }
}

// A group of result tiles (GRP x 16 columns at n0; `cnt` of them real) -> D.
// Lane (m, g) holds row m, columns 16i + g + 4v of tile i.  Staged: written
// into the wave's region (16 rows x 512 bytes, 16-byte chunks XOR-swizzled by
// row), read back as 2 rows x 512 bytes per store.
// ncols: D's true width, where the kernel takes tails (columns past it are
// not written).
template <class C>
__device__ __forceinline__ void gen64_store_group(unsigned char* lds, int stg, const d4_t (&acc)[C::GRP], int cnt,
                                                  __amdgpu_buffer_rsrc_t rs, int64_t ldd, int n0, int lane,
                                                  int ncols = 0) {
    const int m = lane & 15, g = lane >> 4;
    if (stg < 0) {
#pragma unroll
        for (int i = 0; i < C::GRP; ++i)
            if (i < cnt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int col = n0 + 16 * i + g + 4 * v;
                    const u2_t x = dsplit(acc[i][v]);
                    if (!C::TAIL || col < ncols)
                        __builtin_amdgcn_raw_buffer_store_b64(x, rs, (int)((m * ldd + col) * 8), 0, 0);
                }
        return;
    }
    unsigned char* st = lds + stg;
#pragma unroll
    for (int i = 0; i < C::GRP; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int col = 16 * i + g + 4 * v, ch = col >> 1;
            *(double*)(st + m * 512 + ((ch ^ m) << 4) + (col & 1) * 8) = acc[i][v];
        }
    asm volatile("" ::: "memory");   // one wave's LDS accesses complete in order
    const int q = lane & 31, nq = 8 * cnt;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int r = 2 * k + (lane >> 5);
        const u4_t x = *(const u4_t*)(st + r * 512 + ((q ^ r) << 4));
        if (q < nq) {
            const int col = n0 + 2 * q;
            if constexpr (C::TAIL) st_pair64(rs, (uint32_t)((r * ldd + col) * 8), x, ncols - col, false);
            else st128(rs, (uint32_t)((r * ldd + col) * 8), x);
        }
    }
    asm volatile("" ::: "memory");
}

// One GEMM on one wave's 16 rows: x holds ks operand K-steps; nt result tiles
// of 16 columns, GRP at a time (the last group repeats its last tile and drops
// the copies); sink(t, acc, cnt) takes each group.
template <class C, bool FIRST, class Sink>
__device__ __forceinline__ void gen64_gemm(const unsigned char* lds, const Gen64Frag& fr, const double (&x)[C::MKS],
                                           int ks, int nt, Sink&& sink) {
    ks = uniform_here(ks);
    nt = uniform_here(nt);
#pragma unroll
    for (int t = 0; t < C::MNT; t += C::GRP) {
        if (t < nt) {
            d4_t acc[C::GRP];
            int ti[C::GRP];
#pragma unroll
            for (int i = 0; i < C::GRP; ++i) ti[i] = t + i < nt ? t + i : nt - 1;
            // K-step 0 always exists: its products start from zero, with no
            // accumulator to clear
#pragma unroll
            for (int i = 0; i < C::GRP; ++i)
                acc[i] = Ty<DT_F64>::mma(gen64_wfrag<FIRST>(lds, fr, ti[i], 0), x[0], d4_t{0.0, 0.0, 0.0, 0.0});
#pragma unroll
            for (int j = 1; j < C::MKS; ++j)
                if (j < ks)
#pragma unroll
                    for (int i = 0; i < C::GRP; ++i)
                        acc[i] = Ty<DT_F64>::mma(gen64_wfrag<FIRST>(lds, fr, ti[i], j), x[j], acc[i]);
            sink(t, acc, nt - t < C::GRP ? nt - t : C::GRP);
        }
    }
}

template <int B, int E, class F>
__device__ __forceinline__ void gen64_static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        gen64_static_for<B + 1, E>(f);
    }
}

template <class C>
__device__ __forceinline__ void gen64_body(const KArgs& args) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // d: the widths the kernel lays out (padded where it takes tails); dt: true
    int d[C::NST + 1], dt[C::NST + 1];
#pragma unroll
    for (int i = 0; i <= C::NST; ++i) {
        dt[i] = args.dims[i];
        d[i] = !C::TAIL ? dt[i] : i == 0 ? (dt[i] + 7) / 8 * 8 : (dt[i] + 15) / 16 * 16;
    }
    Gen64Frag fr[C::NST];
    int off = 0;
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        fr[s].init(off, d[s], s == 0, lane);
        off += d[s] * d[s + 1] * 8;
    }
    const int ks0 = d[0] / 4, dn = d[C::NST];
    const int stg = gen64_stage_d(d, C::NST) ? off + wave * C::STG : -1;

    const int G = gridDim.x, bid = blockIdx.x;
    const int lid = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
    const int per = args.total_tiles / G, extra = args.total_tiles % G;
    const int t0 = lid * per + (lid < extra ? lid : extra);
    const int t1 = t0 + per + (lid < extra ? 1 : 0);
    if (t0 >= t1) return;
    const int TB = args.tiles_per_batch;
    // the first segment's weight copies go out before the entry arithmetic
    if constexpr (!C::TAIL) gen64_copy_weights<C>(lds, d, args, t0 / TB, wave);
    __builtin_amdgcn_sched_barrier(0);

    int t_end = t1;
    auto rows_of = [&](int t) {
        const int64_t row0 = (int64_t)(t % TB) * C::ROWS_WG + wave * C::ROWS_WAVE;
        const int64_t r = args.M - row0;
        return r < 0 ? (int64_t)0 : (r > C::ROWS_WAVE ? (int64_t)C::ROWS_WAVE : r);
    };
    auto a_rsrc = [&](int t) {
        const bool live = t < t_end;
        const int tc = live ? t : t0;
        const int64_t rows = live ? rows_of(tc) : 0;
        const int64_t row0 = (int64_t)(tc % TB) * C::ROWS_WG + wave * C::ROWS_WAVE;
        return make_rsrc((const char*)args.A + ((int64_t)(tc / TB) * args.sA + (rows ? row0 : 0) * args.lda) * 8,
                         (uint32_t)(rows * args.lda * 8));
    };

    auto process = [&](int t, const double (&a)[C::MKS]) __attribute__((always_inline)) {
        const int64_t rows = rows_of(t), row0 = (int64_t)(t % TB) * C::ROWS_WG + wave * C::ROWS_WAVE;
        const auto d_rs = make_rsrc((char*)args.D + ((int64_t)(t / TB) * args.sD + (rows ? row0 : 0) * args.ldd) * 8,
                                    (uint32_t)(rows * args.ldd * 8));
        auto to_d = [&](int tt, const d4_t (&acc)[C::GRP], int cnt) __attribute__((always_inline)) {
            gen64_store_group<C>(lds, stg, acc, cnt, d_rs, args.ldd, 16 * tt, lane, dt[C::NST]);
        };
        if constexpr (C::NST == 1) {
            gen64_gemm<C, true>(lds, fr[0], a, ks0, dn / 16, to_d);
        } else {
            // the operands of stage s come from oA (s odd) or oB (s even, s > 0):
            // K-step 4t + v is register v of result tile t
            double oA[C::MKS], oB[C::MKS];
            auto to_ops = [&](double (&o)[C::MKS]) __attribute__((always_inline)) {
                return [&o](int tt, const d4_t (&acc)[C::GRP], int cnt) __attribute__((always_inline)) {
#pragma unroll
                    for (int i = 0; i < C::GRP; ++i)
                        if (i < cnt)
#pragma unroll
                            for (int v = 0; v < 4; ++v) o[4 * (tt + i) + v] = acc[i][v];
                };
            };
            gen64_gemm<C, true>(lds, fr[0], a, ks0, d[1] / 16, to_ops(oA));
            gen64_static_for<1, C::NST - 1>([&](auto sc) __attribute__((always_inline)) {
                constexpr int S = decltype(sc)::value;
                if constexpr (S % 2 == 1) gen64_gemm<C, false>(lds, fr[S], oA, d[S] / 4, d[S + 1] / 16, to_ops(oB));
                else gen64_gemm<C, false>(lds, fr[S], oB, d[S] / 4, d[S + 1] / 16, to_ops(oA));
            });
            constexpr int L = C::NST - 1;
            if constexpr (L % 2 == 1) gen64_gemm<C, false>(lds, fr[L], oA, d[L] / 4, dn / 16, to_d);
            else gen64_gemm<C, false>(lds, fr[L], oB, d[L] / 4, dn / 16, to_d);
        }
    };

    const auto no_rsrc = make_rsrc(args.A, 0u);
    double ring[C::PF + 1][C::MKS];
    int t = t0;
    bool issued = !C::TAIL;   // the first segment's weights are on their way
    while (t < t1) {
        const int b = t / TB;
        t_end = (b + 1) * TB < t1 ? (b + 1) * TB : t1;
        auto load = [&](double (&a)[C::MKS], int tt) __attribute__((always_inline)) {
            if constexpr (C::TAIL) gen64_load_a_tail<C>(a, a_rsrc(tt), args.lda, ks0, dt[0], lane);
            else gen64_load_a<C>(a, a_rsrc(tt), no_rsrc, args.lda, ks0, lane);
        };
        if constexpr (C::TAIL) {
            __syncthreads();   // the previous segment's weight reads are over
            gen64_stage_weights_tail<C>(lds, d, dt, args, b);
            __syncthreads();
            load(ring[0], t);
        } else {
            if (!issued) {
                __syncthreads();   // the previous segment's weight reads are over
                gen64_copy_weights<C>(lds, d, args, b, wave);
            }
            issued = false;
            // the segment's first A tile goes out behind the weights; both
            // are waited for here (the copies are not the compiler's to wait for)
            load(ring[0], t);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        if constexpr (C::PF == 0) {
            for (;;) {
                process(t, ring[0]);
                if (++t >= t_end) break;
                load(ring[0], t);
            }
        } else {
            for (;;) {
                load(ring[1], t + 1);
                process(t, ring[0]);
                if (++t >= t_end) break;
                load(ring[0], t + 1);
                process(t, ring[1]);
                if (++t >= t_end) break;
            }
        }
    }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void gen64_kernel(KArgs args) {
    gen64_body<C>(args);
}

}  // namespace b2bk
