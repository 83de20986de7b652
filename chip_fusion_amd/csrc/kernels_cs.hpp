// Column-split fused kernel for cascades whose weights exceed LDS (e.g. two
// 256 x 256 bf16 matrices, 256 KB).
//
// Page 1 ("数据处理方法、装置、设备及介质", detailed description) also performs
// the rearrangement in shared memory: the warp writes its results to shared
// memory, they are rearranged there and read back in the layout the next
// operator needs.  Here that is the natural form: the four waves of a
// workgroup each own a quarter of the columns of every GEMM and keep that
// quarter of the weights in registers; the intermediate C0 of a 32-row tile
// is assembled in LDS from the four column slices (rounded to the input
// type) and read back by every wave as the operand of the second GEMM -- the
// relation between the first GEMM's result layout and the second GEMM's
// operand layout is realised by the LDS addresses.  Nothing leaves the chip.
//
// The weights are first re-laid out by a small kernel into fragment order in
// a workspace (every workgroup needs all of them; reading them as contiguous
// 16-byte fragments avoids staging 256 KB through LDS in every workgroup).
// Per 32-row tile: A is loaded with whole-row 16-byte accesses into LDS
// (XOR-swizzled 16-byte chunks), GEMM0 (each wave: 32 rows x N1/4 columns),
// C0 -> LDS, GEMM1 (each wave: 32 rows x N2/4 columns), D -> LDS, row-wise
// stores.  Three workgroup barriers per tile.
#pragma once
#include "kernels.hpp"

namespace b2bk {

template <int DT_, int K_, int N1_, int N2_, int PF_ = 2>
struct CsCfg {
    static constexpr int DT = DT_, K = K_, N1 = N1_, N2 = N2_, PF = PF_;
    static constexpr int WAVES = 4, THREADS = 256, MT = 2, R = 32;
    static constexpr int ELT = Ty<DT>::ELT;
    static_assert(DT != DT_F64, "column split is written for 16-bit types");
    static constexpr int N1W = N1 / WAVES, N2W = N2 / WAVES;   // per-wave column slices
    static constexpr int NT0 = N1W / 16, NT1 = N2W / 16;       // 16-column tiles per slice
    static constexpr int KS0 = K / 32, KS1 = N1 / 32;           // K-steps of each GEMM
    static constexpr int ABYTES = R * K * ELT, CBYTES = R * N1 * ELT, DBYTES = R * N2 * ELT;
    static constexpr int LDS_TILES = ABYTES + CBYTES + DBYTES;
    static constexpr int LDS_BYTES = LDS_TILES;
    static constexpr int A_CHUNKS = ABYTES / 16 / THREADS;      // 16-byte A loads per thread per tile
    static_assert(N1W % 32 == 0 && N2W % 32 == 0, "column slices must be whole 32-column pairs");
    static_assert(ABYTES % (16 * THREADS) == 0, "A tile must split evenly over the threads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS");
    // row-major tiles in LDS, 16-byte chunks XOR-swizzled by row (conflict-free
    // column reads of 16 consecutive rows)
    __device__ static inline int apos(int row, int chunk) { return row * K * ELT + ((chunk ^ (row & 15)) << 4); }
    __device__ static inline int cpos(int row, int chunk) { return row * N1 * ELT + ((chunk ^ (row & 15)) << 4); }
    __device__ static inline int dpos(int row, int chunk) { return row * N2 * ELT + ((chunk ^ (row & 15)) << 4); }
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

template <class C>
__global__ __launch_bounds__(256) void cs_pack_kernel(KArgs args, u4_t* ws, int64_t batch) {
    using P = Packed<C>;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= batch * P::PER_BATCH) return;
    const int64_t b = gid / P::PER_BATCH;
    int sl = (int)(gid % P::PER_BATCH);
    const int mat = sl < P::SLOTS0 ? 0 : 1;
    if (mat) sl -= P::SLOTS0;
    const int KS = mat ? C::KS1 : C::KS0;
    const int f = sl >> 6, l = sl & 63, t = f / KS, ks = f % KS, i = l & 15, g = l >> 4;
    const unsigned short* B = (const unsigned short*)args.B[mat] + b * args.sB[mat] + 16 * t + i;
    const int64_t ldb = args.ldb[mat];
    unsigned h[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) h[u] = B[(int64_t)(32 * ks + 8 * g + u) * ldb];
    ws[gid] = u4_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

template <class C>
__device__ __forceinline__ void cs_body(const KArgs& args) {
    using T = Ty<C::DT>;
    __shared__ __attribute__((aligned(16))) unsigned char lds[C::LDS_BYTES];
    unsigned char* const lA = lds;
    unsigned char* const lC = lds + C::ABYTES;
    unsigned char* const lD = lds + C::ABYTES + C::CBYTES;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, g = lane >> 4;

    const int G = gridDim.x, bid = blockIdx.x;
    const int lid = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
    const int per = args.total_tiles / G, extra = args.total_tiles % G;
    const int t0 = lid * per + (lid < extra ? lid : extra);
    const int t1 = t0 + per + (lid < extra ? 1 : 0);
    if (t0 >= t1) return;
    const int TB = args.tiles_per_batch;

    // weights of this wave's column slices, in registers
    u4_t w0[C::NT0][C::KS0], w1[C::NT1][C::KS1];

    // A tile of 32 rows: thread loads chunks tid + i*256 of the row-major tile
    int t_end = t1;
    auto a_rsrc = [&](int t) {
        const bool live = t < t_end;
        const int tc = live ? t : t0;
        const int b = tc / TB;
        const int64_t row0 = (int64_t)(tc % TB) * C::R;
        int64_t rows = args.M - row0;
        rows = rows < 0 ? 0 : (rows > C::R ? C::R : rows);
        if (!live) rows = 0;
        const char* base = (const char*)args.A + ((int64_t)b * args.sA + (rows ? row0 : 0) * args.lda) * C::ELT;
        return make_rsrc(base, (uint32_t)(rows * args.lda * C::ELT));
    };
    constexpr int CPR_A = C::K * C::ELT / 16;   // 16-byte chunks per row of A
    auto load_tile = [&](u4_t (&r)[C::A_CHUNKS], int t) {
        const auto rs = a_rsrc(t);
#pragma unroll
        for (int i = 0; i < C::A_CHUNKS; ++i) {
            const int j = tid + i * C::THREADS, row = j / CPR_A, c = j % CPR_A;
            r[i] = ld128(rs, (uint32_t)(row * args.lda * C::ELT + c * 16));
        }
    };
    auto write_tile = [&](const u4_t (&r)[C::A_CHUNKS]) {
#pragma unroll
        for (int i = 0; i < C::A_CHUNKS; ++i) {
            const int j = tid + i * C::THREADS, row = j / CPR_A, c = j % CPR_A;
            *(u4_t*)(lA + C::apos(row, c)) = r[i];
        }
    };

    auto process = [&](int t) {
        const int b = t / TB;
        const int64_t row0 = (int64_t)(t % TB) * C::R;
        int64_t rows = args.M - row0;
        rows = rows < 0 ? 0 : (rows > C::R ? C::R : rows);

        // GEMM0 on this wave's N1 slice: C0^T = W0^T . A^T, A fragments from LDS
        f4_t acc0[C::MT][C::NT0];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int n = 0; n < C::NT0; ++n) acc0[mt][n] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < C::KS0; ++ks) {
            u4_t a[C::MT];
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt) a[mt] = *(const u4_t*)(lA + C::apos(16 * mt + m, 4 * ks + g));
#pragma unroll
            for (int n = 0; n < C::NT0; ++n)
#pragma unroll
                for (int mt = 0; mt < C::MT; ++mt) acc0[mt][n] = T::mma(w0[n][ks], a[mt], acc0[mt][n]);
        }
        // round, regroup pairs of tiles to 8 consecutive columns per lane, assemble C0 in LDS
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int c = 0; c < C::NT0 / 2; ++c) {
                const f4_t x = acc0[mt][2 * c], y = acc0[mt][2 * c + 1];
                unsigned x0 = T::pack(x[0], x[1]), x1 = T::pack(x[2], x[3]);
                unsigned y0 = T::pack(y[0], y[1]), y1 = T::pack(y[2], y[3]);
                regroup_pairs(x0, x1, y0, y1);
                const int chunk = (wave * C::N1W + 32 * c + 8 * g) / 8;
                *(u4_t*)(lC + C::cpos(16 * mt + m, chunk)) = u4_t{x0, x1, y0, y1};
            }
        __syncthreads();   // C0 complete (all four slices)

        // GEMM1 on this wave's N2 slice, C0 rows read back as the operand
        f4_t acc1[C::MT][C::NT1];
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int n = 0; n < C::NT1; ++n) acc1[mt][n] = f4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < C::KS1; ++kc) {
            u4_t o[C::MT];
#pragma unroll
            for (int mt = 0; mt < C::MT; ++mt) o[mt] = *(const u4_t*)(lC + C::cpos(16 * mt + m, 4 * kc + g));
#pragma unroll
            for (int n = 0; n < C::NT1; ++n)
#pragma unroll
                for (int mt = 0; mt < C::MT; ++mt) acc1[mt][n] = T::mma(w1[n][kc], o[mt], acc1[mt][n]);
        }
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
#pragma unroll
            for (int c = 0; c < C::NT1 / 2; ++c) {
                const f4_t x = acc1[mt][2 * c], y = acc1[mt][2 * c + 1];
                unsigned x0 = T::pack(x[0], x[1]), x1 = T::pack(x[2], x[3]);
                unsigned y0 = T::pack(y[0], y[1]), y1 = T::pack(y[2], y[3]);
                regroup_pairs(x0, x1, y0, y1);
                const int chunk = (wave * C::N2W + 32 * c + 8 * g) / 8;
                *(u4_t*)(lD + C::dpos(16 * mt + m, chunk)) = u4_t{x0, x1, y0, y1};
            }
        __syncthreads();   // D complete; every wave is done with A and C0

        // whole-row stores: wave w writes rows 8w .. 8w+7
        const auto d_rs = make_rsrc(
            (char*)args.D + ((int64_t)b * args.sD + (rows ? row0 : 0) * args.ldd) * C::ELT,
            (uint32_t)(rows * args.ldd * C::ELT));
        constexpr int CPR_D = C::N2 * C::ELT / 16;
        constexpr int ROWS_PER_WAVE = C::R / C::WAVES;
#pragma unroll
        for (int i = 0; i < ROWS_PER_WAVE * CPR_D / 64; ++i) {
            const int j = i * 64 + lane, row = wave * ROWS_PER_WAVE + j / CPR_D, c = j % CPR_D;
            const u4_t v = *(const u4_t*)(lD + C::dpos(row, c));
            st128(d_rs, (uint32_t)(row * args.ldd * C::ELT + c * 16), v);
        }
    };

    constexpr int RING = C::PF + 1;
    u4_t ring[RING][C::A_CHUNKS];
    int t = t0;
    while (t < t1) {
        const int b = t / TB;
        t_end = (b + 1) * TB < t1 ? (b + 1) * TB : t1;
        // weights of batch b: this wave's column slices, straight from the
        // pre-packed workspace (contiguous 16-byte loads, no LDS, no barrier);
        // the A prefetch below is issued behind them
        {
            using P = Packed<C>;
            const auto wrs = make_rsrc((const u4_t*)args.W + (int64_t)b * P::PER_BATCH,
                                       (uint32_t)(P::PER_BATCH * 16));
            __syncthreads();   // previous segment's LDS reads are over
#pragma unroll
            for (int n = 0; n < C::NT0; ++n)
#pragma unroll
                for (int ks = 0; ks < C::KS0; ++ks)
                    w0[n][ks] = ld128(wrs, (uint32_t)((((wave * C::NT0 + n) * C::KS0 + ks) * 64 + lane) * 16));
#pragma unroll
            for (int n = 0; n < C::NT1; ++n)
#pragma unroll
                for (int kc = 0; kc < C::KS1; ++kc)
                    w1[n][kc] = ld128(wrs, (uint32_t)((P::SLOTS0 + ((wave * C::NT1 + n) * C::KS1 + kc) * 64 + lane) * 16));
        }
#pragma unroll
        for (int i = 0; i < C::PF; ++i) load_tile(ring[i], t + i);
        // A tiles: registers hold the next PF tiles; the current one is written
        // to LDS once every wave is done with the previous tile
        for (;;) {
            bool done = false;
#pragma unroll
            for (int ph = 0; ph < RING; ++ph) {
                if (!done) {
                    __syncthreads();   // previous tile's A/C0/D reads are over
                    write_tile(ring[ph]);
                    load_tile(ring[(ph + C::PF) % RING], t + C::PF);
                    __syncthreads();   // A tile in LDS
                    process(t);
                    done = ++t >= t_end;
                }
            }
            if (done) break;
        }
    }
}

template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 1)))
void cs_kernel(KArgs args) {
    cs_body<C>(args);
}

}  // namespace b2bk
