/*
 * b2b.h -- C ABI of the fused cascaded ("back-to-back") GEMM library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page 1, "数据处理方法、装置、设备及介质", detailed description:
 * the definition of cascaded GEMM as several GEMM operators fused into one,
 * and the note that three or more operators may be fused):
 *
 *     D[b] = rnd( rnd( A[b] . B0[b] ) . B1[b] )                 (N3 == 0)
 *     D[b] = rnd( rnd( rnd( A[b] . B0[b] ) . B1[b] ) . B2[b] )   (N3 >  0)
 *
 * for b in [0, batch).  Nothing sits between the operators (no scale, bias or
 * activation; the pages fuse operators whose output feeds the next input
 * directly).  Accumulation is float32 for fp16/bf16 inputs and float64 for
 * fp64; rnd rounds to nearest-even into the input type (identity for fp64).
 * The intermediates never leave the chip: the first GEMM's accumulator
 * fragment is rearranged in registers (cross-lane exchange) or through LDS
 * into the operand layout of the next GEMM (page 1: the rearrangement
 * relation, the coordination matrix of Fig. 4, and the shared-memory variant).
 *
 * Shapes: A is M x K, B0 is K x N1, B1 is N1 x N2, B2 is N2 x N3, D is M x N_last
 * (N_last = N3 if N3 > 0 else N2).  All matrices are row-major with leading
 * dimensions in elements; batches are strided by batch_stride elements
 * (0 broadcasts a weight matrix to every batch; A and D must not use 0).
 *
 * Ownership: the caller owns every matrix and the stream.  A plan owns only
 * host tables and, with B2B_FLAG_UNFUSED, a device workspace for the
 * intermediates that b2b_gemm_create allocates and b2b_gemm_destroy frees
 * (b2b_gemm_run rewrites it on every call, so two unfused runs of one plan
 * that overlap on different streams race; fused runs share no memory).
 *
 * Errors: every call returns a status and never aborts; on failure of create
 * *plan is set to NULL.  b2b_gemm_run only enqueues work on the stream and
 * never synchronises; launch failures are reported as B2B_ERROR_HIP, faults
 * inside a kernel are not detectable at the call.
 */
#ifndef B2B_H_
#define B2B_H_

#include <hip/hip_runtime_api.h> /* hipStream_t */
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    B2B_DTYPE_F16 = 0,   /* IEEE binary16 inputs and outputs, float32 accumulation */
    B2B_DTYPE_BF16 = 1,  /* bfloat16 inputs and outputs, float32 accumulation */
    B2B_DTYPE_F64 = 2,   /* binary64 throughout */
    B2B_DTYPE_TF32 = 3,  /* the type of page 1's worked example: binary32 inputs,
                            intermediates and outputs; every GEMM rounds both operands
                            to tf32 (10 fraction bits, nearest-even), multiplies them
                            and sums the products in binary32.  gfx950 has no tf32
                            matrix instruction: each tf32 operand is split exactly into
                            two bfloat16 parts and a product takes three bf16 passes
                            (the part product of the two low parts, below 2^-14 of
                            the product, dropped) or, with B2B_FLAG_TF32_EXACT, four
                            (every product exact).  Run-time widths on the 32x32x16
                            instruction: K and every N multiples of 32, each at most
                            128, weights at most 160 KB at 4 bytes per element; one to
                            three GEMMs fused, any number unfused; rearrangement
                            RELABEL.  Non-finite inputs (and values that round past
                            the largest tf32 value) give NaN where tf32 arithmetic
                            would give an infinity. */
    B2B_DTYPE_FP8_E4M3 = 4 /* OCP fp8 E4M3 (bias 7, largest value 448, no infinities),
                            one byte per element: only as the type of the second GEMM
                            of a two-GEMM b2b_chain_create_typed cascade (its B1 and the
                            intermediate, rounded to nearest-even on chip; results
                            beyond 448 in magnitude after rounding give NaN).  The
                            second GEMM runs on v_mfma_scale_f32_32x32x64_f8f6f4 with
                            unit scales, products exact, sums in float32. */
} b2b_dtype_t;

typedef enum {
    B2B_SUCCESS = 0,
    B2B_ERROR_INVALID_VALUE = 1,  /* bad dimension, leading dimension, pointer or alignment */
    B2B_ERROR_NOT_SUPPORTED = 2,  /* the cascade cannot be fused with this dtype/shape/mode */
    B2B_ERROR_HIP = 3,            /* a HIP runtime call failed */
    B2B_ERROR_OUT_OF_MEMORY = 4,  /* host or device allocation failed */
    B2B_ERROR_WORKSPACE_LIMIT = 5 /* b2b_chain_run_static: the intermediates need more than
                                     B2B_STATIC_WORKSPACE_BYTES */
} b2b_status_t;

/* Flags of b2b_gemm_create. */
enum {
    B2B_FLAG_UNFUSED = 1u << 0,    /* comparison path: one GEMM kernel per operator, the
                                      rounded intermediates go through HBM */
    B2B_FLAG_ORIENT_N = 1u << 1,   /* first GEMM computed as A.B0 (accumulator lanes hold
                                      columns); default computes it transposed so that lanes
                                      hold rows.  Only with REMAP_BPERMUTE or REMAP_LDS. */
    B2B_FLAG_TF32_EXACT = 1u << 3, /* tf32 only: four bf16 passes per product instead of three */
    B2B_FLAG_MFMA_32X32 = 1u << 2, /* fp16/bf16 only: kernels on v_mfma_f32_32x32x16 with the
                                      widths taken at run time (K, N1..N3 multiples of
                                      32, each at most 256, the fused path's weights at most
                                      160 KB; the unfused path's per GEMM).  Rearrangement
                                      REMAP_RELABEL (the default) or REMAP_PERMLANE (a swap of
                                      32-lane halves).  Without this flag these kernels serve
                                      fp16/bf16 cascades that no fixed-width kernel covers; fp64
                                      cascades no fixed-width kernel covers go to fp64 kernels
                                      with run-time widths (v_mfma_f64_16x16x4; K a multiple of
                                      8, N1..N3 of 16, each at most 128, weights at most 160 KB;
                                      the layouts coincide, nothing moves). */
    B2B_REMAP_AUTO = 0u << 4,      /* the library picks the rearrangement */
    B2B_REMAP_BPERMUTE = 1u << 4,  /* coordination-matrix rounds: one ds_bpermute per round */
    B2B_REMAP_PERMLANE = 2u << 4,  /* fixed lane-row swaps (v_permlane16/32_swap) */
    B2B_REMAP_LDS = 3u << 4,       /* through a wave-private LDS region */
    B2B_REMAP_RELABEL = 4u << 4,   /* no data movement: the next GEMM's K order follows the
                                      accumulator layout */
    B2B_REMAP_MASK = 7u << 4
};

typedef struct b2b_gemm_plan* b2b_gemm_t;   /* opaque, owned by the library */

/*
 * Plans a cascade (page 1: determining the operators to fuse and the
 * rearrangement relation between them, done once on the host).
 *   plan          out: the new plan, or NULL on failure
 *   dtype         element type of A, B*, D
 *   batch, M      batch count and rows of A / D (M may be any positive value)
 *   K, N1, N2     inner dimensions; N3 = 0 for two GEMMs, > 0 for three
 *   ld            leading dimensions in elements: {lda, ldb0, ldb1, ldb2, ldd};
 *                 NULL means dense (ld = number of columns); ldb2 ignored if N3 == 0
 *   batch_stride  batch strides in elements: {A, B0, B1, B2, D}; NULL means dense;
 *                 0 for a B* broadcasts it
 *   flags         B2B_FLAG_* | B2B_REMAP_*
 * Widths and layouts: K, N1, N2 (, N3) may be any positive values and the
 * leading dimensions and batch strides any values at least the row width
 * (page 1 derives the relation for whatever operators are adjacent; nothing
 * ties it to a size granule).  Cascades whose widths are whole granules of
 * the instructions (fp16/bf16: multiples of 32; fp64: K of 8, N of 16) and
 * whose rows and batches start on 16-byte boundaries run on the kernels
 * described with the flags; the others -- one type throughout (fp16, bf16
 * or fp64), rearrangement AUTO or RELABEL -- run on kernels that pad every
 * width to the granule on chip (zero weights in LDS, zero columns of A past
 * K, D's columns past N not written), fused when the padded widths stay
 * within the run-time-width bounds (fp16/bf16: 256 and the weights within
 * LDS, one to three GEMMs; fp64: 64 for two or three GEMMs), unfused
 * otherwise (one GEMM a kernel, fp16/bf16 to 256, fp64 to 128).
 * Returns INVALID_VALUE for non-positive sizes, ld below the row width, ld
 * or a batch stride off a 16-byte multiple on a cascade the padding kernels
 * do not take (a type per stage, tf32, fp8, orientation N, a rearrangement
 * other than RELABEL), a leading dimension whose span over 32 rows of
 * A or D, or over all rows of a weight matrix, reaches 2^31 bytes (the
 * kernels' buffer offsets are 32-bit), unknown flags, or more than 2^31 - 1 row tiles
 * (batch x ceil(M / rows a workgroup takes)); NOT_SUPPORTED for cascades no
 * kernel covers: padded widths beyond the bounds above, a tail on a cascade
 * the padding kernels do not take, or weights beyond LDS (then the caller may
 * retry with B2B_FLAG_UNFUSED, whose per-GEMM kernels need only one matrix in
 * LDS).
 */
b2b_status_t b2b_gemm_create(b2b_gemm_t* plan, b2b_dtype_t dtype, int64_t batch, int64_t M,
                             int64_t K, int64_t N1, int64_t N2, int64_t N3,
                             const int64_t* ld, const int64_t* batch_stride, uint32_t flags);

/*
 * Executes a planned cascade (page 1: the rearrangement module of the
 * apparatus, Fig. 5, i.e. the execution step of the method's flow in Fig. 1:
 * the operators run fused, the first one's result rearranged on chip into
 * the second one's operand by the relation the plan fixed).
 * Enqueues the cascade on `stream` (NULL is the null stream).
 * A, B0, B1, B2, D are device pointers, 16-byte aligned; B2 must be NULL iff
 * N3 == 0; D must not alias any input.  Only enqueues; does not synchronise.
 * Plans of one GEMM or of more than three (b2b_chain_create) take
 * b2b_chain_run; here they return INVALID_VALUE.
 */
b2b_status_t b2b_gemm_run(b2b_gemm_t plan, const void* A, const void* B0, const void* B1,
                          const void* B2, void* D, hipStream_t stream);

/*
 * A cascade of any number of GEMMs (page 1 allows as many fused operators as
 * the flow holds): D = rnd(...rnd(rnd(A.B_0).B_1)...B_{nst-1}).
 *   nst           GEMMs, 1..8
 *   widths        nst + 1 values: K, then the column count of every B_s (the
 *                 last is D's)
 *   ld            nst + 2 leading dimensions in elements: A, B_0..B_{nst-1},
 *                 D; NULL means dense
 *   batch_stride  nst + 2 batch strides in elements, same order; NULL means
 *                 dense; 0 for a B_s broadcasts it
 *   flags         as for b2b_gemm_create
 * Up to three GEMMs this plans exactly what b2b_gemm_create plans.  Longer
 * fused cascades run on the run-time-width kernels (fp16/bf16 up to eight GEMMs,
 * K and the widths multiples of 32, each at most 256, or 128 for seven and
 * eight GEMMs; fp64 up to five, each at
 * most 64; all weights together at most 160 KB); the unfused path takes any
 * cascade whose single GEMMs are covered.  Errors as for b2b_gemm_create; INVALID_VALUE also for nst outside
 * 1..8 or a NULL widths.
 */
b2b_status_t b2b_chain_create(b2b_gemm_t* plan, b2b_dtype_t dtype, int64_t batch, int64_t M, int32_t nst,
                              const int64_t* widths, const int64_t* ld, const int64_t* batch_stride,
                              uint32_t flags);

/*
 * A cascade with a type per stage (page 1: each fused operator may
 * have its own data type, and the rearrangement relation follows the type):
 * GEMM s multiplies X_s by B_s in dtypes[s] with fp32 accumulation, and its
 * result is rounded to nearest-even into dtypes[s + 1], the next GEMM's
 * operand type; D is in dtypes[nst].
 *   dtypes        nst + 1 types: A and B_0 in dtypes[0], B_s in dtypes[s],
 *                 D in dtypes[nst]; B2B_DTYPE_F16 or B2B_DTYPE_BF16 (the
 *                 same type throughout, fp64 included, plans exactly what
 *                 b2b_chain_create plans)
 *   other arguments as for b2b_chain_create
 * Mixed types run relabelled on the 32x32x16 run-time-width kernels: fused
 * for two or three GEMMs (widths up to 256) and four to eight (up to 128), all
 * weights together within 160 KB, and unfused for any length (each GEMM then
 * changes type on its way out).  NOT_SUPPORTED for fp64
 * mixed with a 16-bit type, B2B_FLAG_ORIENT_N, a rearrangement other than
 * RELABEL or AUTO, or widths those kernels do not cover; otherwise errors as
 * for b2b_chain_create.  Runs with b2b_chain_run (or b2b_gemm_run for two or
 * three GEMMs).
 */
/* An fp8 stage: dtypes = {t0, B2B_DTYPE_FP8_E4M3, tD} with t0, tD fp16 or bf16
 * and nst = 2 -- the first GEMM in t0, its result rounded to fp8 and
 * multiplied by the fp8 B1 on the fp8 instruction, D in tD; K a multiple of 32,
 * N1 of 64, N2 of 32, each at most 256, B0 (2 bytes an element) and B1 (one)
 * within 160 KB.  With B2B_FLAG_UNFUSED the first GEMM writes its result as
 * E4M3 bytes to a workspace and a second kernel multiplies them (the same
 * values and order of sums: D equals the fused result bit for bit). */
b2b_status_t b2b_chain_create_typed(b2b_gemm_t* plan, const b2b_dtype_t* dtypes, int64_t batch, int64_t M,
                                    int32_t nst, const int64_t* widths, const int64_t* ld,
                                    const int64_t* batch_stride, uint32_t flags);

/* Executes a cascade planned by either create call (page 1: the
 * rearrangement module of Fig. 5, the execution step of Fig. 1, for any
 * number of fused operators); B holds its nst weight pointers (device,
 * 16-byte aligned, none equal to D).  Same asynchrony and errors as
 * b2b_gemm_run. */
b2b_status_t b2b_chain_run(b2b_gemm_t plan, const void* A, const void* const* B, void* D, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * unfused path of b2b_chain_create(..., B2B_FLAG_UNFUSED) followed by
 * b2b_chain_run, in one call that allocates nothing -- no device memory, no
 * host heap.  The same single-GEMM kernels run in the same order, so D equals
 * that plan's D bit for bit.  The intermediates go to a workspace the library
 * holds in a device array of B2B_STATIC_WORKSPACE_BYTES (one per GPU it runs
 * on, in device memory from the first call on that GPU until the process
 * ends): intermediate s in half s % 2 of it, or all of it when there is one.
 *   dtype, batch, M, nst, widths, ld, batch_stride   as for b2b_chain_create
 *   A, B, D, stream                                  as for b2b_chain_run
 * Every call on a GPU shares that GPU's array and leaves its last
 * intermediates in it: calls that overlap on one GPU (on different streams,
 * or from several threads) race and must be serialised by the caller.
 * Errors: as b2b_chain_create and b2b_chain_run (the plan is made and dropped
 * inside the call); WORKSPACE_LIMIT when the intermediates need more than the
 * array (the largest times two with three GEMMs or more, each rounded up to
 * 256 bytes, or the only one with two GEMMs); HIP if the array's address
 * cannot be obtained.  Nothing is written to D on an error.
 */
#define B2B_STATIC_WORKSPACE_BYTES (32u << 20)
b2b_status_t b2b_chain_run_static(b2b_dtype_t dtype, int64_t batch, int64_t M, int32_t nst, const int64_t* widths,
                                  const int64_t* ld, const int64_t* batch_stride, const void* A,
                                  const void* const* B, void* D, hipStream_t stream);

/* Releases a plan (and its workspace, after the device is idle). NULL is a no-op. */
b2b_status_t b2b_gemm_destroy(b2b_gemm_t plan);

/* Static description of a status code. */
const char* b2b_status_string(b2b_status_t s);

/*
 * Picks, for this plan, the fastest of the compiled kernels that compute its
 * cascade (both instruction shapes and every rearrangement when the plan was
 * made with B2B_REMAP_AUTO; only the requested ones otherwise).  The caller
 * hands in nsets buffer sets, representative of its use: A[i], the nst
 * weight pointers B[i * nst .. i * nst + nst - 1] and D[i].  In three
 * interleaved rounds every candidate runs once untimed and then `reps` times
 * back to back over the sets in turn (timed with events on `stream`); the
 * median round scores it.  Sets larger together than the 256 MB Infinity
 * Cache time cold HBM traffic, as a stream of distinct batches sees it; a
 * single small set times warm caches.  The planned kernel stays unless
 * another scores at least 3 % faster.  Every D holds the kept kernel's result
 * when the call returns (the call synchronises the stream).  Not for unfused
 * plans (NOT_SUPPORTED).  It changes the plan: no other call may use the plan
 * meanwhile.  reps: 1..10000.
 */
b2b_status_t b2b_gemm_tune(b2b_gemm_t plan, int32_t nsets, const void* const* A, const void* const* B,
                           void* const* D, hipStream_t stream, int32_t reps);

/* Writes a one-line description of the plan (kernel, MFMA shape, orientation,
   remap mode, tile, grid, LDS and workspace bytes, kernel launches per run,
   whether the kernel pads widths on chip, whether its widths are compiled
   in or read at run time, and the width bound of a run-time-width kernel,
   0 for the fixed-width ones) into buf as space-separated key=value pairs,
   NUL-terminated and cut to len - 1 characters. */
b2b_status_t b2b_gemm_get_info(b2b_gemm_t plan, char* buf, size_t len);

/* ------------------------------------------------------------------------- */
/* Rearrangement tables (page 1: the relation between the first and second
 * rearrangement group matrices, Figs. 2a/2b/3, and the coordination matrix of
 * Fig. 4 with its per-round encoding).  Host-only calls, no GPU needed.       */
/* ------------------------------------------------------------------------- */

/* gfx950 matrix-instruction shapes whose layouts the library knows. */
typedef enum {
    B2B_SHAPE_F16_16X16X32 = 0,
    B2B_SHAPE_BF16_16X16X32 = 1,
    B2B_SHAPE_F16_32X32X16 = 2,
    B2B_SHAPE_BF16_32X32X16 = 3,
    B2B_SHAPE_F16_16X16X16 = 4,
    B2B_SHAPE_F64_16X16X4 = 5,
    B2B_SHAPE_FP8_32X32X64 = 6   /* b2b_mfma_probe only (no relation tables) */
} b2b_shape_t;

/*
 * The relation of one remap unit: for the cascade computed with `shape` in
 * orientation `orient_n` (0: first GEMM transposed, 1: plain), the unit holds
 * one M-tile and the smallest run of intermediate columns that is whole
 * accumulator tiles and whole K-steps of the next GEMM.  Element e of lane l
 * is index l*E + e; source element e = tile*C + reg, destination element
 * e = kstep*S + slot.  rel[d] = source index feeding destination index d.
 *   rel       out, capacity `cap` entries (may be NULL to query sizes)
 *   n_out     out: 64*E
 *   elems     out: E, elements per lane
 */
b2b_status_t b2b_remap_relation(b2b_shape_t shape, int orient_n, int32_t* rel, int64_t cap,
                                int64_t* n_out, int32_t* elems);

/*
 * The coordination matrix the device exchange executes, at the granularity
 * the executor moves (`packed` = 1: 32-bit pairs of 16-bit values, possible
 * only where the relation keeps pairs together; 0: single elements).
 * For round j and receiver lane i (index j*64 + i): p = sender lane, q =
 * element the sender gives, r = destination element of the receiver.
 *   p, q, r   out, capacity `cap` each (NULL to query)
 *   rounds    out: number of rounds (= elements per lane at that granularity)
 */
b2b_status_t b2b_remap_schedule(b2b_shape_t shape, int orient_n, int packed, int32_t* p,
                                int32_t* q, int32_t* r, int64_t cap, int32_t* rounds);

/*
 * Remap compiler (page 1's general method, for any pair of layouts): the
 * relation and the coordination rounds between two layouts of the same
 * 64*E elements, each layout given as one label per (lane, element), index
 * l*E + e (any int32 labels, e.g. row*width + column of the element).
 *   elems      E, 1..16
 *   src, dst   64*E labels each
 *   rel        out or NULL: 64*E entries, rel[d] = source index feeding d
 *   p, q, r    out or NULL: 64*E entries each, round-major as in
 *              b2b_remap_schedule (sender lane, sender element, own slot)
 *   rounds     out or NULL: E
 * INVALID_VALUE unless both layouts hold the same 64*E distinct labels.
 * Host-only, no GPU needed.
 */
b2b_status_t b2b_remap_compile(int32_t elems, const int32_t* src, const int32_t* dst, int32_t* rel, int32_t* p,
                               int32_t* q, int32_t* r, int32_t* rounds);

/*
 * Executes coordination rounds (host tables p, q, r as b2b_remap_compile
 * writes them) on one wave: 64*E 32-bit elements `in` (device, index l*E + e)
 * are rearranged into `out` (device), one ds_bpermute per round.
 * INVALID_VALUE unless rounds == elems (1..16), every round asks each lane
 * once and every lane fills each of its slots once.
 */
b2b_status_t b2b_remap_execute(int32_t elems, int32_t rounds, const int32_t* p, const int32_t* q, const int32_t* r,
                               const uint32_t* in, uint32_t* out, hipStream_t stream);

/*
 * Runs one device rearrangement executor on index payloads and writes what
 * it produced (a probe of the exchange kernels, used by the parity tests).
 *   in   device, 64*E source elements (uint16 for 16-bit shapes, uint64 for
 *        fp64), indexed as in b2b_remap_relation
 *   out  device, 64*E destination elements, same type
 *   mode B2B_REMAP_BPERMUTE / PERMLANE / LDS / RELABEL (RELABEL copies the
 *        accumulator registers unchanged, which is what it feeds the MFMA)
 * Only the shapes the fused kernels use are accepted (16x16x32 f16/bf16,
 * 16x16x4 f64); orient_n requires BPERMUTE or LDS.
 */
b2b_status_t b2b_remap_probe(b2b_shape_t shape, int orient_n, uint32_t mode, const void* in,
                             void* out, hipStream_t stream);

/*
 * Runs one matrix instruction of `shape` on raw operand registers and writes
 * every lane's accumulator registers (a probe of the layout catalogue).
 *   a, b  device, 64 lanes x operand elements (8 x 16-bit, 1 x fp64, or
 *         32 x fp8 E4M3 bytes) each
 *   c     device, 64 lanes x accumulator elements (4 x float32, 16 x float32 for
 *         32x32x16 and 32x32x64, or 4 x fp64)
 * Accumulators start at zero.  Shapes: 16x16x32 and 32x32x16 f16/bf16, 16x16x4
 * f64, 32x32x64 fp8 (E4M3 operands, unit scales).
 */
b2b_status_t b2b_mfma_probe(b2b_shape_t shape, const void* a, const void* b, void* c, hipStream_t stream);

/*
 * The kernels' fp32 -> fp8 E4M3 conversion (v_cvt_pk_fp8_f32, used to round
 * the intermediate of an fp8 second GEMM) applied to 256 values: a probe of
 * its rounding against the format's definition.
 *   x  device, 256 float32;  y  device, 256 bytes (the codes in order)
 */
b2b_status_t b2b_fp8_convert_probe(const float* x, void* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* B2B_H_ */
