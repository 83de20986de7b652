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
// The weights are first re-laid out by a small kernel into fragment order in
// a workspace (every workgroup needs all of them; reading them as contiguous
// 16-byte fragments avoids staging 256 KB through LDS in every workgroup).
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
    static constexpr int LDS_BYTES = OFF_D + YW * DSLICE;
    static constexpr int A_LOADS = ABYTES / (16 * 64 * XW);      // 1 KB loads per first-GEMM wave per tile
    static constexpr int ROW_A = K * ELT, CPR_A = ROW_A / 16;    // bytes, 16-byte chunks per row of A
    static constexpr int ROWS_LOAD = 1024 / ROW_A;               // rows of A per 1 KB load
    static constexpr int DCH = N2W * ELT / 16;                   // 16-byte chunks per row of a D slice
    static_assert(PF >= 1 && N1W % 32 == 0 && N2W % 32 == 0, "column slices must be whole 32-column pairs");
    static_assert(ABYTES % (16 * 64 * XW) == 0 && 1024 % ROW_A == 0 && CPR_A >= 16,
                  "A tile must split into whole 1 KB loads of whole rows");
    static_assert(DCH == 8, "D slices are written as 128-byte row segments");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    static_assert(PF <= 5 && A_LOADS == 4, "wait counts");
    // row-major A and C0 tiles, 16-byte chunks XOR-swizzled by row
    // (conflict-free fragment reads of 16 consecutive rows)
    __device__ static inline int apos(int row, int chunk) { return row * ROW_A + ((chunk ^ (row & 15)) << 4); }
    __device__ static inline int cpos(int row, int chunk) { return row * N1 * ELT + ((chunk ^ (row & 15)) << 4); }
    // D slice: 32 rows x 128 B, chunk swizzled so 16 consecutive rows cover all banks
    __device__ static inline int dpos(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }
};

// ---------------------------------------------------------------------------
// Weight pre-pack: B (row-major) -> fragment-major order in a workspace, one
// 16-byte slot (8 k of one column, natural K order) per lane and fragment, so
// that every wave of the fused kernel loads its weight fragments with plain
// contiguous 16-byte loads.  Slot (fragment f = t*KS + ks, lane l = i + 16g)
// of matrix s, batch b lives at ((b * PER_BATCH) + base_s + f*64 + l) * 16.
// ---------------------------------------------------------------------------
template <class C>
struct Packed {
    static constexpr int SLOTS0 = (C::N1 / 16) * C::KS0 * 64;   // 16-byte slots of B0
    static constexpr int SLOTS1 = (C::N2 / 16) * C::KS1 * 64;
    static constexpr int PER_BATCH = SLOTS0 + SLOTS1;
};

// One workgroup packs a 32 (k) x 64 (n) block of one matrix: coalesced
// 16-byte row loads into LDS, then each thread gathers the 8 k of one column
// for one slot and writes the slots of the block as contiguous 1 KB runs.
template <class C>
struct PackGrid {
    static constexpr int NB0 = C::N1 / 64, NB1 = C::N2 / 64;      // 64-column blocks per matrix
    static constexpr int BLOCKS0 = C::KS0 * NB0, BLOCKS1 = C::KS1 * NB1;
    static constexpr int PER_BATCH = BLOCKS0 + BLOCKS1;           // workgroups per batch
    static_assert(C::N1 % 64 == 0 && C::N2 % 64 == 0, "pack blocks are 64 columns wide");
};

template <class C>
__global__ __launch_bounds__(256) void cs_pack_kernel(KArgs args, u4_t* ws, int64_t batch) {
    using P = Packed<C>;
    using PG = PackGrid<C>;
    constexpr int PITCH = 64 + 4;                                  // halfs per LDS row (padded)
    __shared__ unsigned short tile[32 * PITCH];
    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x / PG::PER_BATCH;
    int blk = blockIdx.x % PG::PER_BATCH;
    const int mat = blk < PG::BLOCKS0 ? 0 : 1;
    if (mat) blk -= PG::BLOCKS0;
    const int NB = mat ? PG::NB1 : PG::NB0, KS = mat ? C::KS1 : C::KS0;
    const int ks = blk / NB, nb = blk % NB;
    const unsigned short* B = (const unsigned short*)args.B[mat] + b * args.sB[mat];
    const int64_t ldb = args.ldb[mat];
    {
        const int r = tid >> 3, c = tid & 7;                       // row of the block, 8-column chunk
        const u4_t v = *(const u4_t*)(B + (int64_t)(32 * ks + r) * ldb + 64 * nb + 8 * c);
        unsigned short* d = tile + r * PITCH + 8 * c;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d[2 * i] = (unsigned short)(v[i] & 0xFFFFu);
            d[2 * i + 1] = (unsigned short)(v[i] >> 16);
        }
    }
    __syncthreads();
    const int t = tid >> 6, l = tid & 63, i = l & 15, g = l >> 4;  // slot: tile t of the block, lane l
    unsigned h[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) h[u] = tile[(8 * g + u) * PITCH + 16 * t + i];
    const int f = (4 * nb + t) * KS + ks;                          // fragment (16-column tile, K-step)
    ws[b * P::PER_BATCH + (mat ? P::SLOTS0 : 0) + f * 64 + l] =
        u4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// Workgroup barrier with explicit waits: "s_waitcnt" for the given counts,
// then s_barrier.  The A ring is written by buffer loads that go straight to
// LDS and complete through vmcnt, so the wait for the tile needed next is
// written out (the tiles behind it stay in flight); the asm also keeps the
// compiler from moving memory accesses across the barrier.
#define B2B_BARRIER_VM(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")
#define B2B_BARRIER() asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory")

template <int N> struct VmWait;
#define B2B_VMWAIT(n) template <> struct VmWait<n> { __device__ static inline void barrier() { B2B_BARRIER_VM(n); } };
B2B_VMWAIT(0) B2B_VMWAIT(2) B2B_VMWAIT(4) B2B_VMWAIT(6) B2B_VMWAIT(8) B2B_VMWAIT(10) B2B_VMWAIT(12)
B2B_VMWAIT(16) B2B_VMWAIT(20) B2B_VMWAIT(24) B2B_VMWAIT(28) B2B_VMWAIT(32)
#undef B2B_VMWAIT

// Barrier that first waits until at most `tiles` A tiles (L loads each) of
// this wave are still in flight; `tiles` is uniform, 0 <= tiles <= 4.
template <int L>
__device__ inline void barrier_tiles_in_flight(int tiles) {
    switch (tiles) {
        case 0: VmWait<0>::barrier(); break;
        case 1: VmWait<L>::barrier(); break;
        case 2: VmWait<2 * L>::barrier(); break;
        case 3: VmWait<3 * L>::barrier(); break;
        default: VmWait<4 * L>::barrier(); break;
    }
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <class C>
__device__ __forceinline__ void cs_body(const KArgs& args) {
    using T = Ty<C::DT>;
    using P = Packed<C>;
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
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (lds_ptr_t)(dst + q * 1024), 16, row * (int)args.lda * C::ELT + chunk * 16, 0, 0,
                kStreamPolicy);
        }
    };

    int t = t0;
    while (t < t1) {
        const int b = t / TB;
        t_end = (b + 1) * TB < t1 ? (b + 1) * TB : t1;
        const int nseg = t_end - t;
        B2B_BARRIER();   // the previous segment's LDS reads are over
        {
            // this wave's weight fragments, straight from the pre-packed workspace
            const auto wrs = make_rsrc((const u4_t*)args.W + (int64_t)b * P::PER_BATCH,
                                       (uint32_t)(P::PER_BATCH * 16));
            const int base = first ? 0 : P::SLOTS0;
#pragma unroll
            for (int n = 0; n < C::NT0; ++n)
#pragma unroll
                for (int ks = 0; ks < C::KS0; ++ks)
                    w[n][ks] = ld128(wrs, (uint32_t)((base + ((sw * C::NT0 + n) * C::KS0 + ks) * 64 + lane) * 16));
        }
        // A prefetch depth ramps up: tiles 0..last(-1) before the first step,
        // then up to two more per step until PF tiles are ahead.  Issuing all
        // PF tiles at once delays tile 0 (every workgroup asks for its whole
        // ring at the same moment and the memory system serves them
        // interleaved); tile 0 first lets the pipeline start about as soon
        // as the weights are in.
        auto last = [&](int s) { return s < 0 ? (C::PF - 1 < 1 ? C::PF - 1 : 1) : (2 * s + 3 < s + C::PF ? 2 * s + 3 : s + C::PF); };
        if (first) {
            for (int k = 0; k <= last(-1); ++k) load_tile(t + k, k);
            barrier_tiles_in_flight<C::A_LOADS>(last(-1));   // tile 0 of the segment is in LDS
        } else {
            // the weights are this wave's only loads: wait for them here, in a
            // form the compiler sees, so it adds no full wait at the step loop
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
            B2B_BARRIER();
        }
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
                B2B_BARRIER();
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
