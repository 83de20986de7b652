// Column-split fused kernel for cascades whose weights exceed LDS (e.g. two
// 256 x 256 bf16 matrices, 256 KB).
//
// Page 1 ("数据处理方法、装置、设备及介质", detailed description) also performs
// the rearrangement in shared memory: results are written to shared memory,
// rearranged there and read back in the layout the next operator needs.  Here
// that is the natural form.  A workgroup has eight waves, two per SIMD: four
// "first-GEMM" waves each own a quarter of the columns of B0, four
// "second-GEMM" waves a quarter of the columns of B1, every wave keeping its
// quarter of the weights in registers.  The intermediate C0 of a 32-row tile
// is assembled in LDS from the four column slices (rounded to the input type)
// and read back by every second-GEMM wave as its operand -- the relation
// between the first GEMM's result layout and the second GEMM's operand layout
// is realised by the LDS addresses.  Nothing leaves the chip.
//
// The two halves work as a two-stage pipeline, one workgroup barrier per
// step: in step s the first-GEMM waves compute C0 of tile s while the
// second-GEMM waves compute D of tile s-1 from the other C0 buffer, so each
// SIMD always has two independent MFMA streams.  A tiles stream straight from
// HBM into a ring of LDS slots (buffer loads that write LDS, whole-row
// accesses, XOR-swizzled 16-byte chunks), several tiles ahead, without
// passing through registers.  Each second-GEMM wave stages its 32 x 64 slice
// of D in a private LDS region and writes it as whole 128-byte row segments.
//
// The weights reach the registers through LDS at the start of each batch
// segment: 64-row chunks of B0 and B1 are copied row-major into LDS (buffer
// loads that write LDS, four chunks in flight, in the space the A ring, the
// C0 buffers and the D slices use later), and each wave picks its fragments out of them
// with transposing LDS reads (ds_read_b64_tr_b16: a 4 x 16 block of 16-bit
// values comes back one column per lane), so the MFMA operand's K-contiguous
// layout needs no separate re-layout pass over the weights.
#pragma once
#include "kernels.hpp"

namespace b2bk {

template <int DT_, int K_, int N1_, int N2_, int NA_ = 6>
struct CsCfg {
    static constexpr int DT = DT_, K = K_, N1 = N1_, N2 = N2_;
    static constexpr int NA = NA_, PF = NA_ - 1;               // A slots in LDS; tiles in flight
    static constexpr int XW = 4, YW = 4;                        // first- and second-GEMM waves
    static constexpr int WAVES = XW + YW, THREADS = 64 * WAVES, MT = 2, R = 32;
    static constexpr int ELT = Ty<DT>::ELT;
    static_assert(DT != DT_F64, "column split is written for 16-bit types");
    static constexpr int N1W = N1 / XW, N2W = N2 / YW;          // per-wave column slices
    static constexpr int NT0 = N1W / 16, NT1 = N2W / 16;        // 16-column tiles per slice
    static constexpr int KS0 = K / 32, KS1 = N1 / 32;            // K-steps of each GEMM
    static constexpr int ABYTES = R * K * ELT, CBYTES = R * N1 * ELT, DSLICE = R * N2W * ELT;
    static constexpr int OFF_C = NA * ABYTES, OFF_D = OFF_C + 2 * CBYTES;
    static constexpr int A_LOADS = ABYTES / (16 * 64 * XW);      // 1 KB loads per first-GEMM wave per tile
    static constexpr int ROW_A = K * ELT, CPR_A = ROW_A / 16;    // bytes, 16-byte chunks per row of A
    static constexpr int ROWS_LOAD = 1024 / ROW_A;               // rows of A per 1 KB load
    static constexpr int DCH = N2W * ELT / 16;                   // 16-byte chunks per row of a D slice
    static_assert(PF >= 1 && N1W % 32 == 0 && N2W % 32 == 0, "column slices must be whole 32-column pairs");
    static_assert(ABYTES % (16 * 64 * XW) == 0 && 1024 % ROW_A == 0 && CPR_A >= 16,
                  "A tile must split into whole 1 KB loads of whole rows");
    static_assert(DCH == 8, "D slices are written as 128-byte row segments");
    static_assert(PF <= 5 && A_LOADS == 4, "wait counts");
    // weight staging: chunks of 64 rows (32 KB) of B0 then B1, row-major, 16-byte
    // chunks swizzled so the transposing fragment reads are conflict-free
    static constexpr int WROWS = 64, WCH = WROWS * N1 * ELT;      // rows and bytes per chunk
    static constexpr int NCH0 = K / WROWS, NCH = NCH0 + N1 / WROWS;
    static constexpr int W_LOADS = WCH / (16 * 64 * WAVES);       // 1 KB loads per wave per chunk
    static constexpr int NWB = 4;                                 // staging buffers = chunks in flight
    // the fourth staging buffer starts at the D slices and runs past them
    static constexpr int LDS_BYTES = (OFF_D + YW * DSLICE > OFF_D + WCH) ? OFF_D + YW * DSLICE : OFF_D + WCH;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(N1 * ELT == 512 && N2 * ELT == 512 && K % WROWS == 0 && N1 % WROWS == 0,
                  "weight staging is written for rows of 512 bytes");
    static_assert(NCH0 == 4 && NCH == 8 && W_LOADS == 4 && NA >= 6,
                  "staging buffers: ring slots 2-3, 4-5, the C0 buffers and the D slices");
    __device__ static inline int wswz(int r) { return 2 * ((r & 3) | (((r >> 3) & 3) << 2)); }
    __device__ static inline int wpos(int r, int chunk) { return r * 512 + ((chunk ^ wswz(r)) << 4); }
    // row-major A and C0 tiles, 16-byte chunks XOR-swizzled by row
    // (conflict-free fragment reads of 16 consecutive rows)
    __device__ static inline int apos(int row, int chunk) { return row * ROW_A + ((chunk ^ (row & 15)) << 4); }
    __device__ static inline int cpos(int row, int chunk) { return row * N1 * ELT + ((chunk ^ (row & 15)) << 4); }
    // D slice: 32 rows x 128 B, chunk swizzled so that the rows one 16-byte
    // store touches -- 8 or 16 consecutive rows, one chunk each, however
    // many lanes the LDS serves a cycle -- and the two rows one read covers
    // fall on distinct banks (the pairing (row >> 1) of an earlier layout
    // put rows 2j and 2j + 1 of a store on one bank: 12 % of LDS-active
    // cycles were conflicts)
    __device__ static inline int dpos(int row, int chunk) {
        return row * 128 + ((chunk ^ ((row & 7) ^ ((row >> 3) & 1))) << 4);
    }
};

template <class C>
__device__ __forceinline__ void cs_body(const KArgs& args) {
    using T = Ty<C::DT>;
    __shared__ __attribute__((aligned(1024))) unsigned char lds[C::LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool first = wave < C::XW;                   // first-GEMM wave
    const int sw = first ? wave : wave - C::XW;        // column slice of this wave
    const int m = lane & 15, g = lane >> 4;

    const int G = gridDim.x, bid = blockIdx.x;
    const int lid = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
    const int per = args.total_tiles / G, extra = args.total_tiles % G;
    const int t0 = lid * per + (lid < extra ? lid : extra);
    const int t1 = t0 + per + (lid < extra ? 1 : 0);
    if (t0 >= t1) return;
    const int TB = args.tiles_per_batch;

    // weights of this wave's column slice (B0 for first-GEMM waves, B1 for
    // second-GEMM waves), in registers
    u4_t w[C::KS0 > C::KS1 ? C::NT0 : C::NT1][C::KS0 > C::KS1 ? C::KS0 : C::KS1];
    static_assert(C::NT0 == C::NT1 && C::KS0 == C::KS1, "both slices hold the same number of fragments");

    auto rows_of = [&](int t) {
        const int64_t row0 = (int64_t)(t % TB) * C::R;
        int64_t rows = args.M - row0;
        return rows < 0 ? (int64_t)0 : (rows > C::R ? (int64_t)C::R : rows);
    };
    // A tile t -> LDS slot (buffer loads that write LDS; empty resource past
    // the segment, so every tile step issues the same number of loads)
    int t_end = t1;
    auto load_tile = [&](int t, int slot) {
        const bool live = t < t_end;
        const int tc = live ? t : t0;
        const int64_t rows = live ? rows_of(tc) : 0;
        const int64_t row0 = (int64_t)(tc % TB) * C::R;
        const char* base = (const char*)args.A +
                           ((int64_t)(tc / TB) * args.sA + (rows ? row0 : 0) * args.lda) * C::ELT;
        const auto rs = make_rsrc(base, (uint32_t)(rows * args.lda * C::ELT));
        unsigned char* dst = lds + slot * C::ABYTES;
#pragma unroll
        for (int j = 0; j < C::A_LOADS; ++j) {
            const int q = sw * C::A_LOADS + j;                       // 1 KB piece of the slot
            const int row = q * C::ROWS_LOAD + lane / C::CPR_A, pos = lane % C::CPR_A;
            const int chunk = pos ^ (row & 15);                      // lands at apos(row, chunk)
            lds_dma16<true>(rs, dst + q * 1024, row * (int)args.lda * C::ELT + chunk * 16);
        }
    };

    // Weights: chunk c (64 rows of B0 for c < 4, of B1 after) goes to staging
    // buffer c % 4 -- ring slots 2-3, ring slots 4-5, the C0 buffers, the D
    // slices -- while ring slots 0-1 receive A tiles 0 and 1.  Order of
    // issue: chunks 0-3, A tiles 0-1 (first-GEMM waves), then chunk c+4 once
    // chunk c has been read.
    auto buf = [&](int c) -> unsigned char* {
        const int i = c % C::NWB;
        return lds + (i == 0 ? 2 * C::ABYTES : i == 1 ? 4 * C::ABYTES : i == 2 ? C::OFF_C : C::OFF_D);
    };
    auto load_chunk = [&](int b, int c) {
        const int mat = c < C::NCH0 ? 0 : 1, c4 = mat ? c - C::NCH0 : c;
        const int64_t rows = mat ? C::N1 : C::K;
        const auto rs = make_rsrc((const char*)args.B[mat] + (int64_t)b * args.sB[mat] * C::ELT,
                                  (uint32_t)(rows * args.ldb[mat] * C::ELT));
        unsigned char* dst = buf(c);
#pragma unroll
        for (int i = 0; i < C::W_LOADS; ++i) {
            const int q = wave * C::W_LOADS + i;                 // 1 KB piece: rows 2q, 2q+1 of the chunk
            const int r = 2 * q + lane / 32, pos = lane % 32;
            const int chunk = pos ^ C::wswz(r);                  // lands at wpos(r, chunk)
            lds_dma16<false>(rs, dst + q * 1024, (int)((C::WROWS * c4 + r) * args.ldb[mat] * C::ELT) + chunk * 16);
        }
    };

    // The first segment's first chunks go out before anything else: the
    // compiler computes the addresses the rest of the kernel needs at entry
    // (~400 instructions a wave, ~1 us), which would otherwise delay them.
    int t = t0;
    bool issued = true;
#pragma unroll
    for (int c = 0; c < C::NWB; ++c) load_chunk(t0 / TB, c);
    __builtin_amdgcn_sched_barrier(0);
    while (t < t1) {
        const int b = t / TB;
        t_end = (b + 1) * TB < t1 ? (b + 1) * TB : t1;
        const int nseg = t_end - t;
        if (!issued) {
            // The previous segment's LDS reads are over, and its A loads past
            // the segment's end have landed: with an empty resource they still
            // write (zeros) into ring slots that this segment's weight chunks,
            // copied by other waves, are about to fill.
            if (first) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            barrier_lds();
#pragma unroll
            for (int c = 0; c < C::NWB; ++c) load_chunk(b, c);
        }
        issued = false;
        // A prefetch depth ramps up: tiles 0..last(-1) before the first step,
        // then up to two more per step until PF tiles are ahead.  Issuing all
        // PF tiles at once delays tile 0 (every workgroup asks for its whole
        // ring at the same moment and the memory system serves them
        // interleaved); tile 0 first lets the pipeline start about as soon
        // as the weights are in.
        auto last = [&](int s) { return s < 0 ? 1 : (2 * s + 3 < s + C::PF ? 2 * s + 3 : s + C::PF); };

        // fragment (16-column tile at n0, 32 rows from k0 of the chunk) of this
        // wave: two transposing reads, rows k0+8g+0..3 and k0+8g+4..7
        auto frag = [&](unsigned char* src, int n0, int k0) {
            const int j = (lane >> 2) & 3, q = lane & 3;
            const int chunk = (n0 >> 3) + (q >> 1);
            u4_t out;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r = k0 + 8 * g + 4 * h + j;
                auto* p = (__attribute__((address_space(3))) unsigned char*)(lds_ptr_t)src +
                          C::wpos(r, chunk) + (q & 1) * 8;
                const tr4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) tr4_t*)p);
                out[2 * h] = ((unsigned)(unsigned short)v[0]) | ((unsigned)(unsigned short)v[1] << 16);
                out[2 * h + 1] = ((unsigned)(unsigned short)v[2]) | ((unsigned)(unsigned short)v[3] << 16);
            }
            return out;
        };
        if (first)
            for (int k = 0; k <= last(-1); ++k) load_tile(t + k, k);
#pragma unroll
        for (int c = 0; c < C::NCH; ++c) {
            // wait for chunk c: chunks min(3, 7 - c) later, and (first-GEMM
            // waves, c <= 3) the two A tiles issued after chunk 3, stay in flight
            static_assert(C::NWB == 4 && C::NCH == 8, "wait counts");
            if (first) {
                if (c <= 3) barrier_vm<3 * C::W_LOADS + 2 * C::A_LOADS>();
                else if (c == 4) barrier_vm<3 * C::W_LOADS>();
                else if (c == 5) barrier_vm<2 * C::W_LOADS>();
                else if (c == 6) barrier_vm<C::W_LOADS>();
                else barrier_vm<0>();
            } else {
                if (c <= 4) barrier_vm<3 * C::W_LOADS>();
                else if (c == 5) barrier_vm<2 * C::W_LOADS>();
                else if (c == 6) barrier_vm<C::W_LOADS>();
                else barrier_vm<0>();
            }
            if (first == (c < C::NCH0)) {
                const int c4 = c < C::NCH0 ? c : c - C::NCH0;
#pragma unroll
                for (int n = 0; n < C::NT0; ++n)
#pragma unroll
                    for (int kl = 0; kl < C::WROWS / 32; ++kl)
                        w[n][(C::WROWS / 32) * c4 + kl] = frag(buf(c), C::N1W * sw + 16 * n, 32 * kl);
            }
            barrier_lds();   // chunk c has been read: its buffer is free
            if (c + C::NWB < C::NCH) load_chunk(b, c + C::NWB);
        }
        // here the weights are in registers and A tiles 0 and 1 are in LDS
        for (int s = 0; s <= nseg; ++s) {
            if (first) {
                if (s < nseg) {
                    for (int k = last(s - 1) + 1; k <= last(s); ++k) load_tile(t + k, k % C::NA);
                    const unsigned char* lA = lds + (s % C::NA) * C::ABYTES;
                    unsigned char* lC = lds + C::OFF_C + (s & 1) * C::CBYTES;
                    // GEMM0 on this wave's N1 slice: C0^T = W0^T . A^T
                    f4_t acc[C::MT][C::NT0];
#pragma unroll
                    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
                        for (int n = 0; n < C::NT0; ++n) acc[mt][n] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < C::KS0; ++ks) {
                        u4_t a[C::MT];
#pragma unroll
                        for (int mt = 0; mt < C::MT; ++mt)
                            a[mt] = *(const u4_t*)(lA + C::apos(16 * mt + m, 4 * ks + g));
#pragma unroll
                        for (int n = 0; n < C::NT0; ++n)
#pragma unroll
                            for (int mt = 0; mt < C::MT; ++mt) acc[mt][n] = T::mma(w[n][ks], a[mt], acc[mt][n]);
                    }
                    // round, regroup pairs of tiles to 8 consecutive columns per lane, C0 slice -> LDS
#pragma unroll
                    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
                        for (int c = 0; c < C::NT0 / 2; ++c) {
                            const f4_t x = acc[mt][2 * c], y = acc[mt][2 * c + 1];
                            unsigned x0 = T::pack(x[0], x[1]), x1 = T::pack(x[2], x[3]);
                            unsigned y0 = T::pack(y[0], y[1]), y1 = T::pack(y[2], y[3]);
                            regroup_pairs(x0, x1, y0, y1);
                            const int chunk = (sw * C::N1W + 32 * c + 8 * g) / 8;
                            *(u4_t*)(lC + C::cpos(16 * mt + m, chunk)) = u4_t{x0, x1, y0, y1};
                        }
                }
                // the next tile's A is complete (this wave's part) before the barrier
                barrier_tiles_in_flight<C::A_LOADS>(last(s) - (s + 1));
            } else {
                if (s >= 1) {
                    const int tt = t + s - 1;
                    const unsigned char* lC = lds + C::OFF_C + ((s - 1) & 1) * C::CBYTES;
                    unsigned char* lD = lds + C::OFF_D + sw * C::DSLICE;
                    // GEMM1 on this wave's N2 slice, full C0 rows read back as the operand
                    f4_t acc[C::MT][C::NT1];
#pragma unroll
                    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
                        for (int n = 0; n < C::NT1; ++n) acc[mt][n] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kc = 0; kc < C::KS1; ++kc) {
                        u4_t o[C::MT];
#pragma unroll
                        for (int mt = 0; mt < C::MT; ++mt)
                            o[mt] = *(const u4_t*)(lC + C::cpos(16 * mt + m, 4 * kc + g));
#pragma unroll
                        for (int n = 0; n < C::NT1; ++n)
#pragma unroll
                            for (int mt = 0; mt < C::MT; ++mt) acc[mt][n] = T::mma(w[n][kc], o[mt], acc[mt][n]);
                    }
                    // round, regroup, stage the 32 x N2W slice in this wave's region
#pragma unroll
                    for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
                        for (int c = 0; c < C::NT1 / 2; ++c) {
                            const f4_t x = acc[mt][2 * c], y = acc[mt][2 * c + 1];
                            unsigned x0 = T::pack(x[0], x[1]), x1 = T::pack(x[2], x[3]);
                            unsigned y0 = T::pack(y[0], y[1]), y1 = T::pack(y[2], y[3]);
                            regroup_pairs(x0, x1, y0, y1);
                            *(u4_t*)(lD + C::dpos(16 * mt + m, 4 * c + g)) = u4_t{x0, x1, y0, y1};
                        }
                    // LDS accesses of one wave complete in order; only the
                    // compiler must not move the reads above the writes
                    asm volatile("" ::: "memory");
                    const int64_t rows = rows_of(tt), row0 = (int64_t)(tt % TB) * C::R;
                    const auto d_rs = make_rsrc(
                        (char*)args.D + ((int64_t)(tt / TB) * args.sD + (rows ? row0 : 0) * args.ldd) * C::ELT,
                        (uint32_t)(rows * args.ldd * C::ELT));
#pragma unroll
                    for (int i = 0; i < C::R * C::DCH / 64; ++i) {
                        const int row = i * (64 / C::DCH) + lane / C::DCH, ch = lane % C::DCH;
                        const u4_t v = *(const u4_t*)(lD + C::dpos(row, ch));
                        st128(d_rs, (uint32_t)((row * args.ldd + sw * C::N2W) * C::ELT + ch * 16), v);
                    }
                }
                barrier_lds();
            }
        }
        t = t_end;
    }
    // the loads issued past the last tile (empty resource) end before the wave
    if (first) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void cs_kernel(KArgs args) {
    cs_body<C>(args);
}

}  // namespace b2bk
