// Fused cascade on the 32x32x16 matrix instruction, with the widths given at
// run time (any multiple of 32 up to the instance's bound).
//
// Page 1 ("数据处理方法、装置、设备及介质", detailed description) derives the
// rearrangement from the register layout of one matrix instruction's result
// and of the next one's operand, per hardware and data type; the same method
// applies to every instruction shape.  On gfx950's v_mfma_f32_32x32x16_{f16,bf16}
// (operand: lane l holds row l%32 and the 8 k values 8*(l/32)+u; result: lane
// l holds column l%32 and rows 8*(v/4) + 4*(l/32) + v%4, v < 16) the first GEMM
// is computed transposed, C0^T = B0^T . A^T, so lane l holds 16 values of row
// l%32 of C0.  The next GEMM's operand (k = 16 per step) needs 8 of them per
// lane:
//   RELABEL   the next GEMM's K order follows the result layout: K-step 2t+s
//             of 32-column tile t takes, in slot u, intermediate column
//             32t + 16s + 8*(u/4) + 4*(l/32) + u%4, which is result register
//             8s+u of the same lane -- nothing moves;
//   PERMLANE  natural K order: the two 32-lane halves trade one 8-byte half of
//             each operand (v_permlane32_swap), two swaps per K-step.
// Nothing leaves the chip between the GEMMs.
//
// Weights live in LDS in blocks of 32 columns (each block all rows x 64
// bytes, so the 4 rows a transposing read touches are 256 contiguous bytes,
// every bank once) and every weight fragment is read with two transposing
// reads (ds_read_b64_tr_b16: a 16-lane group gets a 4 x 16 block back one
// column per lane).  Each wave owns 32 rows of a 256-row tile;
// D is regrouped with the same lane-half swap into 8 consecutive columns per
// lane and stored as 16-byte pieces of rows.
//
// A cascade may give each GEMM its own 16-bit type (GenCfg's type mask):
// the fp16 and bf16 instructions share every register layout, so a stage
// changes only the instruction it issues and the type its result is rounded
// into.
#pragma once
#include "kernels.hpp"

namespace b2bk {

typedef float f16x_t __attribute__((ext_vector_type(16)));

template <int DT> struct Ty32;
template <> struct Ty32<DT_F16> {
    __device__ static inline f16x_t mma(u4_t a, u4_t b, f16x_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(h8_t, a),
                                                      __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
    }
};
template <> struct Ty32<DT_BF16> {
    __device__ static inline f16x_t mma(u4_t a, u4_t b, f16x_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf8_t, a),
                                                       __builtin_bit_cast(bf8_t, b), c, 0, 0, 0);
    }
};

// NST_: GEMMs in the cascade (1 is a single GEMM, for the unfused path; up
// to kMaxStages, the weights of all of them in LDS);
// MAXD_: bound on every width; MODE_: MODE_RELABEL or MODE_PERMLANE;
// PF_: A tiles fetched ahead (0 or 1, registers permitting);
// TM_: -1, every operand, intermediate and D in DT_; else a type per stage
// (page 1 lets each fused operator have its own data type): bit s set means
// bf16, clear fp16, for the operands of GEMM s (A, B_s and the intermediate
// rounded for it) and, at bit NST, for D.  DT_ is then the type of bit 0.
// TM_ = TM_RUNTIME: the same mask read from the kernel arguments (one
// instance for every mixture of a long cascade; each GEMM branches, uniformly,
// to its type's instruction and each rounding selects its type).
// OUT8_: D is written as fp8 E4M3 bytes (the first kernel of an unfused
// cascade whose second GEMM is fp8), else in the last stage's 16-bit type.
constexpr int TM_RUNTIME = -2;

// TAIL_: any widths (the K and N tails of widths that are not multiples of
// 32) and any leading dimensions and batch strides (rows at any element
// alignment): every width is padded to the next multiple of 32 on chip --
// weights zero-filled in LDS, A's columns past K read as zero, D's columns
// past N never written -- so the instructions see a cascade of whole
// granules whose padded rows and columns are exactly zero.
template <int DT_, int NST_, int MAXD_, int MODE_, int PF_, int TM_ = -1, int WAVES_ = 8, bool OUT8_ = false,
          bool TAIL_ = false>
struct GenCfg {
    static constexpr int DT = DT_, NST = NST_, MAXD = MAXD_, MODE = MODE_, PF = PF_, TM = TM_;
    static constexpr bool OUT8 = OUT8_, TAIL = TAIL_;
    static constexpr int DE = OUT8 ? 1 : 2;   // bytes of a D element
    static constexpr bool RTM = TM_ == TM_RUNTIME;
    static constexpr int stype(int s) { return TM < 0 ? DT : (((TM >> s) & 1) ? DT_BF16 : DT_F16); }
    static constexpr int WAVES = WAVES_, THREADS = 64 * WAVES, ROWS_WAVE = 32, ROWS_WG = ROWS_WAVE * WAVES;
    static constexpr int MKS = MAXD / 16, MNT = MAXD / 32;     // K-steps, 32-column tiles
    static constexpr int LDS_MAX = 160 * 1024;
    static_assert(DT != DT_F64, "the 32x32x16 instruction exists for 16-bit types");
    static_assert(MAXD % 32 == 0 && NST >= 1 && NST <= kMaxStages && (PF == 0 || PF == 1), "config");
    static_assert(MODE == MODE_RELABEL || MODE == MODE_PERMLANE, "rearrangement");
    static_assert(TM == -1 || TM == TM_RUNTIME || (TM >= 0 && TM < (2 << NST) && stype(0) == DT), "type mask");
    static_assert(!RTM || MODE == MODE_RELABEL, "run-time types are relabelled");
    static_assert(!TAIL || (TM == -1 && !OUT8 && MODE == MODE_RELABEL), "tails: one type, relabelled");
};

// the widths a kernel lays out: each padded to a multiple of 32 where the
// kernel takes tails, else as given
__host__ __device__ inline void gen_pad(const int32_t* d, int nst, bool tail, int32_t* out) {
    for (int i = 0; i <= nst; ++i) out[i] = tail ? (d[i] + 31) / 32 * 32 : d[i];
}

// One weight matrix in LDS: `rows` x `n` 16-bit values in blocks of 32
// columns, each block `rows` x 64 bytes (row r of block t at t*rows*64 + r*64).
// The 4 consecutive rows a transposing read touches are 256 contiguous bytes,
// all banks once, and a fragment's address steps by constants in the K-step.
struct GenMat {
    int off, rows, n, tstride;
    __device__ inline void init(int off_, int rows_, int n_) {
        off = off_;
        rows = rows_;
        n = n_;
        tstride = rows_ * 64;
    }
    // byte offset of (row r, 16-bit column c)
    __device__ inline int pos(int r, int c) const { return off + (c >> 5) * tstride + r * 64 + ((c & 31) << 1); }
};

// LDS bytes of the weights of a cascade with widths d[0..nst]; with them
// 4 KB per wave (8 waves) of D staging when that still fits the 160 KB
__host__ __device__ inline int64_t gen_weight_bytes(const int32_t* d, int nst) {
    int64_t b = 0;
    for (int s = 0; s < nst; ++s) b += (int64_t)d[s] * d[s + 1] * 2;
    return b;
}
__host__ __device__ inline bool gen_stage_d(const int32_t* d, int nst, int waves = 8) {
    return gen_weight_bytes(d, nst) + waves * 4096 <= 160 * 1024;
}
__host__ __device__ inline int64_t gen_lds_bytes(const int32_t* d, int nst, int waves = 8) {
    return gen_weight_bytes(d, nst) + (gen_stage_d(d, nst, waves) ? waves * 4096 : 0);
}

// Per-lane constants of the weight fragments of one matrix: fragment
// (32-column tile t, K-step j) is read at base[h] + t tstride + 1024 j for
// h = 0, 1 (two transposing reads of 4 rows each).  The K order `rel` is
// false: k = 16j + 8*(l/32) + u, or true: k = 16j + 8*(u/4) + 4*(l/32) + u%4.
struct GenFrag {
    int base[2], tstride;
    __device__ inline void init(const GenMat& m, bool rel, int lane) {
        const int g = lane >> 4, i = lane & 15, jj = i >> 2, q = i & 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int r0 = (rel ? 8 * h + 4 * (g >> 1) : 8 * (g >> 1) + 4 * h) + jj;
            base[h] = m.off + r0 * 64 + 32 * (g & 1) + 8 * q;
        }
        tstride = m.tstride;
    }
};

__device__ __forceinline__ u4_t gen_wfrag(const unsigned char* lds, const GenFrag& fr, int t, int j) {
    u4_t out;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        auto* a = (__attribute__((address_space(3))) unsigned char*)(lds_ptr_t)lds + fr.base[h] + t * fr.tstride +
                  1024 * j;
        const tr4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr4_t*)a);
        out[2 * h] = ((unsigned)(unsigned short)v[0]) | ((unsigned)(unsigned short)v[1] << 16);
        out[2 * h + 1] = ((unsigned)(unsigned short)v[2]) | ((unsigned)(unsigned short)v[3] << 16);
    }
    return out;
}

// A 16-byte chunk of 8 16-bit elements of which `valid` lie inside the
// matrix row (a K or N tail): a whole chunk is one 16-byte load, at any
// element alignment of the row; a partial one is loaded element by element,
// the rest reading as zero, so no access reaches past the row's last element.
__device__ __forceinline__ u4_t ld_chunk16(__amdgpu_buffer_rsrc_t rs, uint32_t off, int valid) {
    if (valid >= 8) return ld128(rs, off);
    u4_t v = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 7; ++e)
        if (e < valid) {
            const unsigned h = (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)(off + 2 * e), 0, 0);
            v[e >> 1] |= h << (16 * (e & 1));
        }
    return v;
}
// the store counterpart: only the chunk's first `valid` elements are written
// (a whole chunk non-temporal unless `part`, i.e. it comes straight from the
// accumulator layout, unstaged; the elements of a partial chunk always with
// the default policy: sent non-temporal, 2-byte stores each went to HBM)
__device__ __forceinline__ void st_chunk16(__amdgpu_buffer_rsrc_t rs, uint32_t off, u4_t v, int valid, bool part) {
    if (valid >= 8) {
        if (part) st128_part(rs, off, v);
        else st128(rs, off, v);
        return;
    }
#pragma unroll
    for (int e = 0; e < 7; ++e)
        if (e < valid)
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(v[e >> 1] >> (16 * (e & 1))), rs,
                                                  (int)(off + 2 * e), 0, 0);
}

// weights of batch b -> LDS, each matrix padded with zeros to the whole
// 32-row, 32-column blocks the kernel lays out (dt: the true widths)
template <class C>
__device__ inline void gen_stage_weights_tail(unsigned char* lds, const GenMat (&mat)[C::NST], const int* dt,
                                              const KArgs& args, int b) {
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        const GenMat& m = mat[s];
        const int rows_t = dt[s], cols_t = dt[s + 1];
        const auto rs = make_rsrc((const char*)args.B[s] + (int64_t)b * args.sB[s] * 2,
                                  (uint32_t)(rows_t * args.ldb[s] * 2));
        const int cpr = m.n / 8, total = m.rows * cpr;
        for (int i0 = 0; i0 < total; i0 += 8 * C::THREADS) {
            u4_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 8;
                const int valid = (i < total && r < rows_t) ? cols_t - c : 0;
                v[k] = ld_chunk16(rs, (uint32_t)((r * args.ldb[s] + c) * 2), valid);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 8;
                if (i < total) *(u4_t*)(lds + m.pos(r, c)) = v[k];
            }
        }
    }
}

// weights of batch b -> LDS (16-byte loads, eight in flight per thread).
// Every thread issues the same loads (past the end: an offset beyond the
// resource, which reads zero), so the compiler's counts of loads in flight
// hold on every path and each LDS write waits for its own load only.
template <class C>
__device__ inline void gen_stage_weights(unsigned char* lds, const GenMat (&mat)[C::NST], const KArgs& args, int b) {
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        const GenMat& m = mat[s];
        const auto rs = make_rsrc((const char*)args.B[s] + (int64_t)b * args.sB[s] * 2,
                                  (uint32_t)(m.rows * args.ldb[s] * 2));
        const int cpr = m.n / 8, total = m.rows * cpr;
        for (int i0 = 0; i0 < total; i0 += 8 * C::THREADS) {
            u4_t v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 8;
                v[k] = ld128(rs, i < total ? (uint32_t)((r * args.ldb[s] + c) * 2) : 0xFFFFFFF0u);
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * C::THREADS + (int)threadIdx.x;
                const int r = i / cpr, c = (i % cpr) * 8;
                if (i < total) *(u4_t*)(lds + m.pos(r, c)) = v[k];
            }
        }
    }
}

// The same copy by buffer loads that write LDS (no registers, nothing to wait
// for before the next instruction): one instruction moves 16 rows x 64 bytes
// of one 32-column block -- lane l takes 16-byte chunk l%4 of row 16i + l/4 --
// which is 1 KB of contiguous LDS in the GenMat layout.  Widths are whole
// blocks here (the tail kernels stage through registers).
template <class C>
__device__ inline void gen_copy_weights(unsigned char* lds, const GenMat (&mat)[C::NST], const KArgs& args, int b,
                                        int wave) {
    const int lane = lane_here();
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        const GenMat& m = mat[s];
        const auto rs = make_rsrc((const char*)args.B[s] + (int64_t)b * args.sB[s] * 2,
                                  (uint32_t)(m.rows * args.ldb[s] * 2));
        const int rg = m.rows / 16, nq = rg * (m.n / 32);
        for (int q = wave; q < nq; q += C::WAVES) {
            const int blk = q / rg, i = q % rg, r = 16 * i + (lane >> 2);
            lds_dma16<false>(rs, lds + m.off + blk * m.tstride + 1024 * i,
                             (int)((r * args.ldb[s] + 32 * blk + 8 * (lane & 3)) * 2));
        }
    }
}

// A fragments of one wave's 32 rows: K-step j holds row l%32, k = 16j + 8*(l/32) + 0..7.
// Two K-steps (64 bytes of a row) come from two loads of 16 rows x 64 bytes
// each -- X: rows 0-15, Y: rows 16-31, lane group g holding 16-byte chunk g
// of the pair -- which two lane swaps turn into the operand layout:
//   X = [X0 X1 X2 X3], Y = [Y0 Y1 Y2 Y3]  (16-lane groups)
//   swap16 -> X = [X0 Y0 X2 Y2], Y = [X1 Y1 X3 Y3]
//   swap32 -> X = [X0 Y0 X1 Y1] (K-step 2p), Y = [X2 Y2 X3 Y3] (K-step 2p+1).
// All loads are issued, those past K through an empty resource (zeros, no
// memory access): the same count on every path keeps the compiler's waits for
// a tile from covering the next tile's loads.
template <class C>
__device__ __forceinline__ void gen_load_a(u4_t (&a)[C::MKS], __amdgpu_buffer_rsrc_t rs,
                                           __amdgpu_buffer_rsrc_t none, int64_t lda, int ks, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int p = 0; p < C::MKS / 2; ++p) {
        const auto src = 2 * p < ks ? rs : none;
        a[2 * p] = ld128(src, (uint32_t)((r * lda + 32 * p + 8 * g) * 2));
        a[2 * p + 1] = ld128(src, (uint32_t)(((16 + r) * lda + 32 * p + 8 * g) * 2));
    }
}

// gen_load_a with a K tail (K: the true width): chunks straddling K are
// loaded element by element, columns past K read as zero
template <class C>
__device__ __forceinline__ void gen_load_a_tail(u4_t (&a)[C::MKS], __amdgpu_buffer_rsrc_t rs, int64_t lda, int ks,
                                                int K, int lane) {
    const int r = lane & 15, g = lane >> 4;
#pragma unroll
    for (int p = 0; p < C::MKS / 2; ++p) {
        const int c0 = 32 * p + 8 * g;
        const int valid = 2 * p < ks ? K - c0 : 0;
        a[2 * p] = ld_chunk16(rs, (uint32_t)((r * lda + c0) * 2), valid);
        a[2 * p + 1] = ld_chunk16(rs, (uint32_t)(((16 + r) * lda + c0) * 2), valid);
    }
}

// the lane swaps of gen_load_a, once the loads have arrived
template <class C>
__device__ __forceinline__ void gen_arrange_a(u4_t (&a)[C::MKS]) {
#pragma unroll
    for (int p = 0; p < C::MKS / 2; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            unsigned x = a[2 * p][i], y = a[2 * p + 1][i];
            swap16(x, y);
            swap32(x, y);
            a[2 * p][i] = x;
            a[2 * p + 1][i] = y;
        }
}

// 16 fp32 values, in pairs, rounded to the 16-bit type NDT, or (NDT < 0) to
// the type `bf` picks at run time: one uniform branch for all of them (a
// select per pair became a branch per pair), on a flag recomputed here
// rather than held as a lane mask
template <int NDT>
__device__ __forceinline__ void gen_pack16(const f16x_t& acc, unsigned (&p)[8], bool bf) {
    if constexpr (NDT >= 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = Ty<NDT>::pack(acc[2 * i], acc[2 * i + 1]);
    } else if (uniform_here(bf ? 1 : 0)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = Ty<DT_BF16>::pack(acc[2 * i], acc[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) p[i] = Ty<DT_F16>::pack(acc[2 * i], acc[2 * i + 1]);
    }
}

// Result tile -> two K-steps of the next GEMM's operand (rounded to its type NDT).
template <class C, int NDT>
__device__ __forceinline__ void gen_to_operand(const f16x_t& acc, u4_t& o0, u4_t& o1, bool bf = false) {
    unsigned p[8];
    gen_pack16<NDT>(acc, p, bf);
    // K-step s: result registers 8s..8s+7 (packed p[4s..4s+3])
    if constexpr (C::MODE == MODE_PERMLANE) {
        // natural K order: half 0 keeps registers 8s..8s+3 and takes the
        // other half's; half 1 keeps 8s+4..8s+7 and takes the other half's
        swap32(p[0], p[2]);
        swap32(p[1], p[3]);
        swap32(p[4], p[6]);
        swap32(p[5], p[7]);
    }
    o0 = u4_t{p[0], p[1], p[2], p[3]};
    o1 = u4_t{p[4], p[5], p[6], p[7]};
}

// Result tiles -> D.  Lane half h of a 32 x 32 result tile holds columns
// 8a + 4h + 0..3; one lane-half swap per pair of blocks leaves 8 consecutive
// columns per lane: n0 + 8h.. and n0 + 16 + 8h.. of row l%32.
template <class C>
__device__ __forceinline__ void gen_regroup_d(const f16x_t& acc, u4_t& lo, u4_t& hi, bool bf = false) {
    constexpr int DDT = C::RTM ? -1 : C::stype(C::NST);
    unsigned p[8];
    gen_pack16<DDT>(acc, p, bf);
    swap32(p[0], p[2]);
    swap32(p[1], p[3]);
    swap32(p[4], p[6]);
    swap32(p[5], p[7]);
    lo = u4_t{p[0], p[1], p[2], p[3]};
    hi = u4_t{p[4], p[5], p[6], p[7]};
}

// A pair of result tiles (64 columns at n0; `two` false: only the first) ->
// D through the wave's 4 KB staging region (32 rows x 128 bytes, 16-byte
// chunks XOR-swizzled by row), read back so that each store writes 8 rows x
// 128 contiguous bytes.  Without a staging region (stg < 0) the 16-byte
// pieces go straight to memory.
// ncols: D's true width, where the kernel takes tails (columns past it are
// not written; chunks straddling it are stored element by element).
template <class C>
__device__ __forceinline__ void gen_store_pair(unsigned char* lds, int stg, const f16x_t& acc0, const f16x_t& acc1,
                                               bool two, __amdgpu_buffer_rsrc_t rs, int64_t ldd, int n0, int lane_,
                                               bool bf = false, int ncols = 0) {
    // From four GEMMs on the lane index passes through an empty asm statement,
    // so that the store offsets are computed here, per tile pair, instead of
    // being held in registers for the whole kernel: the longer chains need
    // those registers (the run-time-typed ones spilled without this; the
    // one-type five-GEMM chain runs 5 % faster).  Shorter cascades keep their
    // offsets (recomputing them cost the three-GEMM run-time-typed instance 7 %).
    int lane = lane_;
    if constexpr (C::NST >= 4) asm volatile("" : "+v"(lane));
    const int m = lane & 31, h = lane >> 5;
    u4_t c[4];
    gen_regroup_d<C>(acc0, c[0], c[1], bf);
    gen_regroup_d<C>(acc1, c[2], c[3], bf);
    if (stg < 0) {
        // chunk q of this lane sits at column n0 + 16 q + 8 h
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (q < 2 || two) {
                const int col = n0 + 16 * q + 8 * h;
                if constexpr (C::TAIL) st_chunk16(rs, (uint32_t)((m * ldd + col) * 2), c[q], ncols - col, true);
                else st128_part(rs, (uint32_t)((m * ldd + col) * 2), c[q]);
            }
        return;
    }
    unsigned char* st = lds + stg;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int chunk = 2 * q + h;                   // 16-byte chunk of the 128-byte row segment
        *(u4_t*)(st + m * 128 + ((chunk ^ (m & 7)) << 4)) = c[q];
    }
    // LDS accesses of one wave complete in order; only the compiler must not
    // move the reads above the writes
    asm volatile("" ::: "memory");
    const int ch = lane & 7, nch = two ? 8 : 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 8 * i + (lane >> 3);
        const u4_t v = *(const u4_t*)(st + r * 128 + ((ch ^ (r & 7)) << 4));
        if (ch < nch) {
            const int col = n0 + 8 * ch;
            if constexpr (C::TAIL) st_chunk16(rs, (uint32_t)((r * ldd + col) * 2), v, ncols - col, false);
            else st128(rs, (uint32_t)((r * ldd + col) * 2), v);
        }
    }
    asm volatile("" ::: "memory");
}

// four fp32 values -> four E4M3 bytes (round to nearest even), x0 lowest
__device__ __forceinline__ int f8_pack4(float x0, float x1, float x2, float x3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// A pair of result tiles -> fp8 D (one byte an element).  Lane (m, h) packs
// columns 8a + 4h + 0..3 of tile q into one dword at byte 32q + 8a + 4h of
// row m's 64-byte segment; through the staging region each store writes 16
// rows x 64 (or 32) contiguous bytes, else the dwords go straight out.
__device__ __forceinline__ void gen_store_pair_f8(unsigned char* lds, int stg, const f16x_t& acc0, const f16x_t& acc1,
                                                  bool two, __amdgpu_buffer_rsrc_t rs, int64_t ldd, int n0, int lane) {
    const int m = lane & 31, h = lane >> 5;
    unsigned w[2][4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        w[0][a] = (unsigned)f8_pack4(acc0[4 * a], acc0[4 * a + 1], acc0[4 * a + 2], acc0[4 * a + 3]);
        w[1][a] = (unsigned)f8_pack4(acc1[4 * a], acc1[4 * a + 1], acc1[4 * a + 2], acc1[4 * a + 3]);
    }
    if (stg < 0) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int a = 0; a < 4; ++a)
                if (q == 0 || two)
                    __builtin_amdgcn_raw_buffer_store_b32(w[q][a], rs, (int)(m * ldd + n0 + 32 * q + 8 * a + 4 * h), 0,
                                                          0);
        return;
    }
    unsigned char* st = lds + stg;
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int a = 0; a < 4; ++a) *(unsigned*)(st + m * 64 + 32 * q + 8 * a + 4 * h) = w[q][a];
    asm volatile("" ::: "memory");
    const int ch = lane & 3, nch = two ? 4 : 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int r = 16 * i + (lane >> 2);
        const u4_t v = *(const u4_t*)(st + r * 64 + 16 * ch);
        if (ch < nch) st128(rs, (uint32_t)(r * ldd + n0 + 16 * ch), v);
    }
    asm volatile("" ::: "memory");
}

// One GEMM of the cascade on one wave's 32 rows: x holds the operand K-steps
// (ks of them), the result has nt tiles of 32 columns, each handed to sink(t, acc).
// Tiles go in pairs: two independent accumulation chains keep the matrix
// core busy while either waits for its previous product.  With an odd tile
// count the last pair computes its tile twice and drops the copy (a branch
// per pair, not per product).  sink(t, acc_t, acc_t+1, two) takes each pair.
// SDT: the GEMM's operand type.
template <class C, int SDT, class Sink>
__device__ __forceinline__ void gen_gemm(const unsigned char* lds, const GenFrag& fr, const u4_t (&x)[C::MKS],
                                         int ks, int nt, Sink&& sink) {
    ks = uniform_here(ks);
    nt = uniform_here(nt);
#pragma unroll
    for (int t = 0; t < C::MNT; t += 2) {
        if (t < nt) {
            const bool two = t + 1 < nt;
            const int t1 = two ? t + 1 : t;
            // K-step 0 always exists (every width is at least 32): its
            // products start from zero, with no accumulator to clear
            f16x_t acc0 = Ty32<SDT>::mma(gen_wfrag(lds, fr, t, 0), x[0], f16x_t{});
            f16x_t acc1 = Ty32<SDT>::mma(gen_wfrag(lds, fr, t1, 0), x[0], f16x_t{});
#pragma unroll
            for (int j = 1; j < C::MKS; ++j)
                if (j < ks) {
                    acc0 = Ty32<SDT>::mma(gen_wfrag(lds, fr, t, j), x[j], acc0);
                    acc1 = Ty32<SDT>::mma(gen_wfrag(lds, fr, t1, j), x[j], acc1);
                }
            sink(t, acc0, acc1, two);
        }
    }
}

// f(integral_constant<int, S>) for S = B .. E-1
template <int B, int E, class F>
__device__ __forceinline__ void gen_static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        gen_static_for<B + 1, E>(f);
    }
}

// The row tiles of one workgroup: a contiguous range of the launch's tiles
// (ROWS_WG rows of one batch each; consecutive workgroups on one XCD, as
// block i runs on XCD i % 8, so a batch's weights are read by one XCD's L2),
// walked one batch segment (one set of weights) at a time.  Everything here
// is uniform across the wave and lives in scalar registers.
template <int ROWS_WG, int ROWS_WAVE>
struct TileRange {
    int t0, t1, TB, t_end, wave;
    int64_t M;
    // false: no tiles for this workgroup
    __device__ inline bool init(const KArgs& a, int wave_) {
        const int G = gridDim.x, bid = blockIdx.x;
        const int lid = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
        const int per = a.total_tiles / G, extra = a.total_tiles % G;
        t0 = lid * per + (lid < extra ? lid : extra);
        t1 = t0 + per + (lid < extra ? 1 : 0);
        TB = a.tiles_per_batch;
        t_end = t1;
        wave = wave_;
        M = a.M;
        return t0 < t1;
    }
    // the tiles from t on that share t's batch
    __device__ inline void segment(int t) {
        const int b = t / TB;
        t_end = (b + 1) * TB < t1 ? (b + 1) * TB : t1;
    }
    __device__ inline int64_t row0(int t) const { return (int64_t)(t % TB) * ROWS_WG + wave * ROWS_WAVE; }
    // this wave's rows of tile t (fewer on the ragged last tile of M, 0 past it)
    __device__ inline int64_t rows(int t) const {
        const int64_t r = M - row0(t);
        return r < 0 ? (int64_t)0 : (r > ROWS_WAVE ? (int64_t)ROWS_WAVE : r);
    }
    // buffer resource over this wave's rows of tile t of a row-major matrix
    // (esz-byte elements, leading dimension ld, batch stride bs)
    __device__ inline __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t ld, int64_t bs, int esz, int t) const {
        const int64_t n = rows(t);
        return make_rsrc((const char*)base + ((int64_t)(t / TB) * bs + (n ? row0(t) : 0) * ld) * esz,
                         (uint32_t)(n * ld * esz));
    }
    // the same for an A tile about to be loaded: past the segment an empty
    // resource, whose loads return zeros without touching memory
    __device__ inline __amdgpu_buffer_rsrc_t a_rsrc(const void* base, int64_t ld, int64_t bs, int esz, int t) const {
        const bool live = t < t_end;
        const int tc = live ? t : t0;
        const int64_t n = live ? rows(tc) : 0;
        return make_rsrc((const char*)base + ((int64_t)(tc / TB) * bs + (n ? row0(tc) : 0) * ld) * esz,
                         (uint32_t)(n * ld * esz));
    }
};

template <class C>
__device__ __forceinline__ void gen_body(const KArgs& args) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // d: the widths the kernel lays out (padded to whole granules where it
    // takes tails); dt: the true widths
    int d[C::NST + 1], dt[C::NST + 1];
#pragma unroll
    for (int i = 0; i <= C::NST; ++i) {
        dt[i] = args.dims[i];
        d[i] = C::TAIL ? (dt[i] + 31) / 32 * 32 : dt[i];
    }
    GenMat mat[C::NST];
    int off = 0;
#pragma unroll
    for (int s = 0; s < C::NST; ++s) {
        mat[s].init(off, d[s], d[s + 1]);
        off += d[s] * d[s + 1] * 2;
    }
    const int ks0 = d[0] / 16, dn = d[C::NST];
    // the wave's D staging region follows the weights, where LDS allows
    const int stg = gen_stage_d(d, C::NST, C::WAVES) ? off + wave * 4096 : -1;

    TileRange<C::ROWS_WG, C::ROWS_WAVE> tr;
    if (!tr.init(args, wave)) return;
    // the first segment's weight copies go out before anything else: the
    // compiler computes the addresses the rest of the kernel needs at entry
    // (several hundred instructions a wave), which would otherwise delay them
    if constexpr (!C::TAIL) gen_copy_weights<C>(lds, mat, args, tr.t0 / tr.TB, wave);
    __builtin_amdgcn_sched_barrier(0);
    constexpr bool REL = C::MODE == MODE_RELABEL;
    GenFrag fr[C::NST];
#pragma unroll
    for (int s = 0; s < C::NST; ++s) fr[s].init(mat[s], REL && s > 0, lane);

    auto a_rsrc = [&](int t) { return tr.a_rsrc(args.A, args.lda, args.sA, 2, t); };

    auto process = [&](int t, const u4_t (&a_in)[C::MKS]) __attribute__((always_inline)) {
        u4_t a[C::MKS];
#pragma unroll
        for (int j = 0; j < C::MKS; ++j) a[j] = a_in[j];
        gen_arrange_a<C>(a);
        const auto d_rs = tr.rsrc(args.D, args.ldd, args.sD, C::DE, t);
        // run-time types: bit s of args.tmask (uniform) picks GEMM s's instruction and
        // the type its result is rounded into for GEMM s+1 (bit NST: D)
        auto bf_at = [&](int s) { return C::RTM && ((uniform_here(args.tmask) >> s) & 1); };
        auto to_d = [&](int tt, const f16x_t& a0, const f16x_t& a1, bool two) __attribute__((always_inline)) {
            if constexpr (C::OUT8) gen_store_pair_f8(lds, stg, a0, a1, two, d_rs, args.ldd, 32 * tt, lane);
            else gen_store_pair<C>(lds, stg, a0, a1, two, d_rs, args.ldd, 32 * tt, lane, bf_at(C::NST), dt[C::NST]);
        };
        // GEMM S on operand x with the sink: its compiled type, or a uniform
        // branch to the type the run-time mask gives
        auto gemm_at = [&](auto sc, const GenFrag& f, const u4_t (&x)[C::MKS], int ks, int nt, auto&& sink)
                           __attribute__((always_inline)) {
            constexpr int S = decltype(sc)::value;
            if constexpr (C::RTM) {
                if (bf_at(S)) gen_gemm<C, DT_BF16>(lds, f, x, ks, nt, sink);
                else gen_gemm<C, DT_F16>(lds, f, x, ks, nt, sink);
            } else {
                gen_gemm<C, C::stype(S)>(lds, f, x, ks, nt, sink);
            }
        };
        using S0 = std::integral_constant<int, 0>;
        if constexpr (C::NST == 1) {
            gemm_at(S0{}, fr[0], a, ks0, dn / 32, to_d);
        } else {
            // the operands of stage s come from oA (s odd) or oB (s even, s > 0),
            // rounded into stage s's type
            u4_t oA[C::MKS], oB[C::MKS];
            auto to_ops = [&](u4_t (&o)[C::MKS], auto nt, bool bf) __attribute__((always_inline)) {
                constexpr int NDT = decltype(nt)::value;
                return [&o, bf](int tt, const f16x_t& a0, const f16x_t& a1, bool two) __attribute__((always_inline)) {
                    gen_to_operand<C, NDT>(a0, o[2 * tt], o[2 * tt + 1], bf);
                    if (two) gen_to_operand<C, NDT>(a1, o[2 * tt + 2], o[2 * tt + 3], bf);
                };
            };
            using T1 = std::integral_constant<int, C::RTM ? -1 : C::stype(1)>;
            gemm_at(S0{}, fr[0], a, ks0, d[1] / 32, to_ops(oA, T1{}, bf_at(1)));
            gen_static_for<1, C::NST - 1>([&](auto sc) __attribute__((always_inline)) {
                constexpr int S = decltype(sc)::value;
                using TN = std::integral_constant<int, C::RTM ? -1 : C::stype(S + 1)>;
                if constexpr (S % 2 == 1)
                    gemm_at(sc, fr[S], oA, d[S] / 16, d[S + 1] / 32, to_ops(oB, TN{}, bf_at(S + 1)));
                else
                    gemm_at(sc, fr[S], oB, d[S] / 16, d[S + 1] / 32, to_ops(oA, TN{}, bf_at(S + 1)));
            });
            constexpr int L = C::NST - 1;
            using SL = std::integral_constant<int, L>;
            if constexpr (L % 2 == 1) gemm_at(SL{}, fr[L], oA, d[L] / 16, dn / 32, to_d);
            else gemm_at(SL{}, fr[L], oB, d[L] / 16, dn / 32, to_d);
        }
    };

    const auto no_rsrc = make_rsrc(args.A, 0u);
    u4_t ring[C::PF + 1][C::MKS];
    int t = tr.t0;
    bool issued = !C::TAIL;   // the first segment's weights are on their way
    while (t < tr.t1) {
        const int b = t / tr.TB;
        tr.segment(t);
        auto load = [&](u4_t (&a)[C::MKS], int tt) __attribute__((always_inline)) {
            if constexpr (C::TAIL) gen_load_a_tail<C>(a, a_rsrc(tt), args.lda, ks0, dt[0], lane);
            else gen_load_a<C>(a, a_rsrc(tt), no_rsrc, args.lda, ks0, lane);
        };
        if constexpr (C::TAIL) {
            __syncthreads();   // the previous segment's weight reads are over
            gen_stage_weights_tail<C>(lds, mat, dt, args, b);
            __syncthreads();
            load(ring[0], t);
        } else {
            if (!issued) {
                __syncthreads();   // the previous segment's weight reads are over
                gen_copy_weights<C>(lds, mat, args, b, wave);
            }
            issued = false;
            // the segment's first A tile goes out behind the weights, and
            // both are waited for here (the copies are not the compiler's to
            // wait for)
            load(ring[0], t);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
        if constexpr (C::PF == 0) {
            for (;;) {
                process(t, ring[0]);
                if (++t >= tr.t_end) break;
                load(ring[0], t);
            }
        } else {
            // two register sets: the next tile's A is in flight while this one is computed
            for (;;) {
                load(ring[1], t + 1);
                process(t, ring[0]);
                if (++t >= tr.t_end) break;
                load(ring[0], t + 1);
                process(t, ring[1]);
                if (++t >= tr.t_end) break;
            }
        }
    }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) void gen_kernel(KArgs args) {
    gen_body<C>(args);
}

// One 32x32x16 instruction on raw operands (64 lanes x 8 16-bit values each),
// all 16 result registers of every lane written out: a probe of the layouts.
template <int DT>
__global__ __launch_bounds__(64) void mfma32_probe_kernel(const void* a, const void* b, void* c) {
    const int lane = threadIdx.x;
    const u4_t av = ((const u4_t*)a)[lane], bv = ((const u4_t*)b)[lane];
    ((f16x_t*)c)[lane] = Ty32<DT>::mma(av, bv, f16x_t{});
}

}  // namespace b2bk
