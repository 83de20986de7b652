/*
 * Plain CPU oracle for the fused cascaded GEMM.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it. It shares no code, header or table with the
 * HIP path.
 *
 * What it computes (page 1, "数据处理方法、装置、设备及介质", detailed
 * description, the cascaded-GEMM definition and the three-operator cascade):
 * a cascade of S = 2 or 3 GEMMs with nothing between them,
 *     X_0 = A,   X_{s+1} = rnd(X_s . B_s),   D = X_S,
 * evaluated independently for every batch and every row.  With a type per
 * stage (oracle_cascade_typed; the pages let each fused operator have its own
 * data type and layout), GEMM s takes X_s and B_s in type t_s and its result is
 * rounded into t_{s+1}, the next GEMM's operand type (t_S is D's type).
 * The 16-bit types serve everywhere; fp8 E4M3 (a format the pages do not
 * name) may be the operand type of a GEMM after the first.  The pages fuse the
 * cascade so that the intermediate never leaves the chip; the value of the
 * cascade itself is the plain matrix product written out here.
 *
 * Readings where the pages are silent:
 *   - accumulation: float32 for fp16/bf16 inputs, float64 for fp64 inputs;
 *     every output element sums its K products in ascending k order from +0;
 *   - rnd: round-to-nearest-even to the input type between stages and for D;
 *     identity for fp64;
 *   - fp64 accumulates with a fused multiply-add per term (C99 fma);
 *   - inputs are dense row-major, batches contiguous.
 *
 * tf32 (the type of the pages' own worked example): inputs and outputs are
 * binary32 values; each GEMM rounds both operands to tf32 (1 sign, 8 exponent
 * and 10 fraction bits: binary32 with the low 13 fraction bits rounded off to
 * nearest-even), multiplies them exactly (two 11-bit significands fit a
 * binary32 product) and sums the K products in binary32, ascending k from +0.
 * The stage result stays binary32 and is rounded to tf32 when the next GEMM
 * takes it as an operand; D is the last stage's binary32 result.
 *
 * The binary16 / bfloat16 encoders below are written from the IEEE 754
 * definitions (round to nearest, ties to even, gradual underflow, overflow to
 * infinity); no vendor conversion routine is used.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared -pthread (no -ffast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F16 = 0, OR_BF16 = 1, OR_F64 = 2, OR_TF32 = 3, OR_FP8 = 4 };

static uint32_t f32_bits(float x) { uint32_t u; memcpy(&u, &x, 4); return u; }
static float bits_f32(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }

/* ---------------------------------------------------------------------------
 * binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * The float's 24-bit significand sig = 1.f (or 0.f for float subnormals) is
 * scaled by 2^(e-23).  The binary16 quantum at magnitude 2^e is 2^(e-10) for
 * e >= -14 (normal range) and 2^-24 below it (subnormal range).  Dropping
 * `sh` low bits of sig and rounding the remainder to nearest-even gives the
 * number of quanta; a carry out of the significand bumps the exponent, which
 * the packed encoding absorbs because exponent and fraction are adjacent.
 * ------------------------------------------------------------------------- */
uint16_t oracle_f32_to_f16(float x)
{
    uint32_t u = f32_bits(x);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t ef = (u >> 23) & 0xFFu;
    uint32_t fr = u & 0x7FFFFFu;
    if (ef == 0xFFu) {                       /* inf or NaN */
        if (fr == 0) return sign | 0x7C00u;
        return sign | 0x7E00u;               /* a quiet NaN */
    }
    if (ef == 0 && fr == 0) return sign;     /* signed zero */
    int e;                                   /* unbiased exponent of the leading bit */
    uint32_t sig;                            /* value = sig * 2^(e-23) */
    if (ef == 0) { e = -126; sig = fr; }     /* float subnormal: 0.f * 2^-126 */
    else { e = (int)ef - 127; sig = fr | 0x800000u; }
    int sh = (e >= -14) ? 13 : (-1 - e);     /* bits below the binary16 quantum */
    uint32_t q, rem, half;
    if (sh >= 32) { q = 0; rem = sig; half = 0xFFFFFFFFu; }  /* far below 2^-25 */
    else {
        q = sig >> sh;
        rem = sig & ((1u << sh) - 1u);
        half = 1u << (sh - 1);
    }
    if (rem > half || (rem == half && (q & 1u))) q++;
    if (e >= -14) {
        /* q in [2^10, 2^11]; encode exponent field e+15 over the leading 1 */
        uint32_t biased = (uint32_t)(e + 15);
        uint32_t enc = (biased << 10) + (q - 0x400u);   /* q = 2^11 carries into the exponent */
        if (enc >= 0x7C00u) return sign | 0x7C00u;      /* overflow -> infinity */
        return sign | (uint16_t)enc;
    }
    /* subnormal range: q quanta of 2^-24; q = 2^10 is the smallest normal */
    return sign | (uint16_t)q;
}

float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h & 0x8000u) << 16;
    uint32_t ef = (h >> 10) & 0x1Fu;
    uint32_t fr = h & 0x3FFu;
    if (ef == 0x1Fu) return bits_f32(sign | 0x7F800000u | (fr << 13));
    if (ef == 0) {                           /* zero or subnormal: fr * 2^-24 exactly */
        float v = (float)fr * 0x1p-24f;
        return sign ? -v : v;
    }
    return bits_f32(sign | ((ef - 15 + 127) << 23) | (fr << 13));
}

/* ---------------------------------------------------------------------------
 * bfloat16: the upper half of a binary32 with the same exponent range; the
 * quantum is 2^16 units of the float's last place everywhere (normal and
 * subnormal alike), so rounding is on the low 16 bits of the encoding.  A
 * carry from the fraction into the exponent field is the correct next binade,
 * and a carry into the all-ones exponent is the correct overflow to infinity.
 * ------------------------------------------------------------------------- */
uint16_t oracle_f32_to_bf16(float x)
{
    uint32_t u = f32_bits(x);
    if (((u >> 23) & 0xFFu) == 0xFFu && (u & 0x7FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);          /* keep NaN a (quiet) NaN */
    uint32_t q = u >> 16, rem = u & 0xFFFFu;
    if (rem > 0x8000u || (rem == 0x8000u && (q & 1u))) q++;
    return (uint16_t)q;
}

float oracle_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* ---------------------------------------------------------------------------
 * tf32: the tf32 quantum is 2^13 units of the binary32 last place in every
 * binade (normal and subnormal alike, the exponent field being the same), so
 * rounding to nearest-even acts on the low 13 bits of the encoding; a carry
 * into the exponent is the next binade, into the all-ones exponent overflow
 * to infinity.  Infinities stay; a NaN stays a (quiet) NaN.
 * ------------------------------------------------------------------------- */
float oracle_round_tf32(float x)
{
    uint32_t u = f32_bits(x);
    if (((u >> 23) & 0xFFu) == 0xFFu) {
        if (u & 0x7FFFFFu) u |= 0x400000u;
        return bits_f32(u & ~0x1FFFu);
    }
    uint32_t q = u >> 13, rem = u & 0x1FFFu;
    if (rem > 0x1000u || (rem == 0x1000u && (q & 1u))) q++;
    return bits_f32(q << 13);
}

void oracle_round_tf32_array(const float* x, float* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_round_tf32(x[i]); }

/* ---------------------------------------------------------------------------
 * fp8 E4M3 (the OCP 8-bit format without infinities): 1 sign bit, 4 exponent
 * bits (bias 7), 3 fraction bits; exponent field 0 holds the subnormals
 * m * 2^-9, the all-ones exponent with fraction 111 is NaN, so the largest
 * value is 1.75 * 2^8 = 448.  Encoding rounds to nearest-even on the quantum
 * 2^(e-3) of the binade 2^e (2^-9 below 2^-6); a result above 448 (any
 * value beyond 464, the half-way point to the odd 480, which would need the
 * NaN code) becomes NaN.
 * ------------------------------------------------------------------------- */
float oracle_fp8_to_f32(uint8_t c)
{
    int sign = c >> 7, ef = (c >> 3) & 0xF, fr = c & 7;
    float v;
    if (ef == 0xF && fr == 7) return sign ? -NAN : NAN;
    if (ef == 0) v = (float)fr * 0x1p-9f;
    else v = ldexpf(1.0f + (float)fr / 8.0f, ef - 7);
    return sign ? -v : v;
}

uint8_t oracle_f32_to_fp8(float x)
{
    uint32_t u = f32_bits(x);
    uint8_t sign = (uint8_t)((u >> 24) & 0x80u);
    if (isnan(x)) return sign | 0x7Fu;
    double a = fabs((double)x);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);                   /* a = f 2^e, 0.5 <= f < 1: leading bit 2^(e-1) */
    int lead = e - 1;
    double quantum = ldexp(1.0, (lead >= -6 ? lead : -6) - 3);
    double q = a / quantum;               /* exact: a power-of-two scaling */
    double fl = floor(q), rem = q - fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = fl * quantum;
    if (r > 448.0) return sign | 0x7Fu;   /* no infinity: NaN */
    if (r < 0x1p-6) return sign | (uint8_t)(r / 0x1p-9);            /* subnormal (or the smallest normal) */
    int re;
    double rf = frexp(r, &re);            /* r = rf 2^re */
    int ef = re - 1 + 7;
    int fr = (int)((rf * 2.0 - 1.0) * 8.0);
    return sign | (uint8_t)((ef << 3) | fr);
}

void oracle_encode_fp8_array(const float* x, uint8_t* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_f32_to_fp8(x[i]); }
void oracle_decode_fp8_array(const uint8_t* x, float* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_fp8_to_f32(x[i]); }

void oracle_encode_f16_array(const float* x, uint16_t* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_f32_to_f16(x[i]); }
void oracle_encode_bf16_array(const float* x, uint16_t* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_f32_to_bf16(x[i]); }
void oracle_decode_f16_array(const uint16_t* x, float* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_f16_to_f32(x[i]); }
void oracle_decode_bf16_array(const uint16_t* x, float* y, int64_t n)
{ for (int64_t i = 0; i < n; ++i) y[i] = oracle_bf16_to_f32(x[i]); }

static float dec16(int dtype, uint16_t h)
{ return dtype == OR_F16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h); }
static uint16_t enc16(int dtype, float x)
{ return dtype == OR_F16 ? oracle_f32_to_f16(x) : oracle_f32_to_bf16(x); }
/* the value of x rounded into a stage type (16-bit or fp8) */
static float round_to(int dtype, float x)
{ return dtype == OR_FP8 ? oracle_fp8_to_f32(oracle_f32_to_fp8(x)) : dec16(dtype, enc16(dtype, x)); }

/* ---------------------------------------------------------------------------
 * One GEMM stage without the final rounding: acc[m][n] = sum_k X[m][k]*B[k][n],
 * k ascending from +0, float32 for 16-bit inputs and float64 (fma) for fp64.
 * X and B are encoded inputs (uint16 bits or doubles); acc is float or double.
 * ------------------------------------------------------------------------- */
int oracle_gemm_acc(int dtype, int64_t M, int64_t K, int64_t N,
                    const void* X, const void* B, void* acc_out)
{
    if (M < 0 || K < 0 || N < 0) return 1;
    if (dtype == OR_F64) {
        const double* x = (const double*)X; const double* b = (const double*)B;
        double* acc = (double*)acc_out;
        for (int64_t m = 0; m < M; ++m) {
            double* row = acc + m * N;
            for (int64_t n = 0; n < N; ++n) row[n] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double a = x[m * K + k];
                for (int64_t n = 0; n < N; ++n) row[n] = fma(a, b[k * N + n], row[n]);
            }
        }
        return 0;
    }
    if (dtype == OR_TF32) {
        const float* x = (const float*)X; const float* b = (const float*)B;
        float* acc = (float*)acc_out;
        for (int64_t m = 0; m < M; ++m) {
            float* row = acc + m * N;
            for (int64_t n = 0; n < N; ++n) row[n] = 0.0f;
            for (int64_t k = 0; k < K; ++k) {
                float a = oracle_round_tf32(x[m * K + k]);
                for (int64_t n = 0; n < N; ++n) row[n] = row[n] + a * oracle_round_tf32(b[k * N + n]);
            }
        }
        return 0;
    }
    if (dtype != OR_F16 && dtype != OR_BF16) return 2;
    const uint16_t* x = (const uint16_t*)X; const uint16_t* b = (const uint16_t*)B;
    float* acc = (float*)acc_out;
    for (int64_t m = 0; m < M; ++m) {
        float* row = acc + m * N;
        for (int64_t n = 0; n < N; ++n) row[n] = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = dec16(dtype, x[m * K + k]);
            for (int64_t n = 0; n < N; ++n) row[n] = row[n] + a * dec16(dtype, b[k * N + n]);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * The whole cascade on a list of rows.  A is [batch][M][dims[0]], B_s is
 * [batch][dims[s]][dims[s+1]], row r of the list selects batch r / M and row
 * r % M; D_out receives the rows of D in list order, [nrows][dims[S]].
 * rows == NULL means every row in order.  Threads split the row list; the
 * arithmetic of each element is the same whatever the split.
 * ------------------------------------------------------------------------- */
#define OR_MAX_STAGES 8

typedef struct {
    int dtype, nst;
    int st[OR_MAX_STAGES + 1];          /* 16-bit type of X_s and B_s; st[nst]: D */
    int64_t batch, M, dims[OR_MAX_STAGES + 1];
    const void* A;
    const float* Bf[OR_MAX_STAGES];     /* decoded weights (16-bit inputs) */
    const double* Bd[OR_MAX_STAGES];    /* weights (fp64 inputs) */
    const int64_t* rows;
    int64_t r0, r1;
    void* D;
    int err;
} job_t;

static void* cascade_worker(void* arg)
{
    job_t* j = (job_t*)arg;
    int64_t wmax = 0;
    for (int s = 0; s <= j->nst; ++s) if (j->dims[s] > wmax) wmax = j->dims[s];
    int is64 = (j->dtype == OR_F64);
    size_t esz = is64 ? sizeof(double) : sizeof(float);
    void* xin = malloc((size_t)wmax * esz);
    void* xout = malloc((size_t)wmax * esz);
    if (!xin || !xout) { j->err = 3; free(xin); free(xout); return NULL; }
    for (int64_t i = j->r0; i < j->r1; ++i) {
        int64_t r = j->rows ? j->rows[i] : i;
        int64_t b = r / j->M, m = r % j->M;
        int64_t K0 = j->dims[0];
        if (is64) {
            const double* a = (const double*)j->A + (b * j->M + m) * K0;
            double* x = (double*)xin;
            for (int64_t k = 0; k < K0; ++k) x[k] = a[k];
            for (int s = 0; s < j->nst; ++s) {
                int64_t K = j->dims[s], N = j->dims[s + 1];
                const double* w = j->Bd[s] + b * K * N;
                double* y = (double*)xout;
                for (int64_t n = 0; n < N; ++n) y[n] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double av = x[k];
                    for (int64_t n = 0; n < N; ++n) y[n] = fma(av, w[k * N + n], y[n]);
                }
                void* t = xin; xin = xout; xout = t; x = (double*)xin;
            }
            memcpy((double*)j->D + i * j->dims[j->nst], xin, (size_t)j->dims[j->nst] * sizeof(double));
        } else if (j->dtype == OR_TF32) {
            const float* a = (const float*)j->A + (b * j->M + m) * K0;
            float* x = (float*)xin;
            for (int64_t k = 0; k < K0; ++k) x[k] = a[k];
            for (int s = 0; s < j->nst; ++s) {
                int64_t K = j->dims[s], N = j->dims[s + 1];
                const float* w = j->Bf[s] + b * K * N;   /* already rounded to tf32 */
                float* y = (float*)xout;
                for (int64_t n = 0; n < N; ++n) y[n] = 0.0f;
                for (int64_t k = 0; k < K; ++k) {
                    float av = oracle_round_tf32(x[k]);
                    for (int64_t n = 0; n < N; ++n) y[n] = y[n] + av * w[k * N + n];
                }
                void* t = xin; xin = xout; xout = t; x = (float*)xin;
            }
            memcpy((float*)j->D + i * j->dims[j->nst], xin, (size_t)j->dims[j->nst] * sizeof(float));
        } else {
            const uint16_t* a = (const uint16_t*)j->A + (b * j->M + m) * K0;
            float* x = (float*)xin;
            for (int64_t k = 0; k < K0; ++k) x[k] = dec16(j->st[0], a[k]);
            uint16_t* drow = (uint16_t*)j->D + i * j->dims[j->nst];
            for (int s = 0; s < j->nst; ++s) {
                int64_t K = j->dims[s], N = j->dims[s + 1];
                const float* w = j->Bf[s] + b * K * N;
                float* y = (float*)xout;
                for (int64_t n = 0; n < N; ++n) y[n] = 0.0f;
                for (int64_t k = 0; k < K; ++k) {
                    float av = x[k];
                    for (int64_t n = 0; n < N; ++n) y[n] = y[n] + av * w[k * N + n];
                }
                /* round the stage result to the next stage's type: this is
                   exactly what the next stage consumes, and what D holds at
                   the end */
                for (int64_t n = 0; n < N; ++n) {
                    if (s + 1 == j->nst) drow[n] = enc16(j->st[s + 1], y[n]);
                    else y[n] = round_to(j->st[s + 1], y[n]);
                }
                void* t = xin; xin = xout; xout = t; x = (float*)xin;
            }
        }
    }
    free(xin); free(xout);
    return NULL;
}

static int cascade_run(int dtype, const int* types, int nstages, const int64_t* dims, int64_t batch,
                       int64_t M, const void* A, const void* const* B, const int64_t* rows,
                       int64_t nrows, void* D_out, int nthreads)
{
    if (nstages < 1 || nstages > OR_MAX_STAGES || batch < 0 || M < 0 || nrows < 0) return 1;
    if (dtype != OR_F16 && dtype != OR_BF16 && dtype != OR_F64 && dtype != OR_TF32) return 2;
    if (types && dtype == OR_TF32) return 2;
    for (int s = 0; s <= nstages; ++s)
        if (types && types[s] != OR_F16 && types[s] != OR_BF16 &&
            !(types[s] == OR_FP8 && s > 0 && s < nstages)) return 2;   /* fp8: operands of a later GEMM */
    for (int s = 0; s <= nstages; ++s) if (dims[s] <= 0) return 1;
    if (!rows) nrows = batch * M;
    if (nrows == 0) return 0;
    if (rows) for (int64_t i = 0; i < nrows; ++i) if (rows[i] < 0 || rows[i] >= batch * M) return 1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if ((int64_t)nthreads > nrows) nthreads = (int)nrows;

    job_t base;
    memset(&base, 0, sizeof base);
    base.dtype = dtype; base.nst = nstages; base.batch = batch; base.M = M;
    for (int s = 0; s <= nstages; ++s) base.dims[s] = dims[s];
    for (int s = 0; s <= nstages; ++s) base.st[s] = types ? types[s] : dtype;
    base.A = A; base.rows = rows; base.D = D_out;
    float* dec[OR_MAX_STAGES] = {0};
    int rc = 0;
    for (int s = 0; s < nstages; ++s) {
        if (dtype == OR_F64) { base.Bd[s] = (const double*)B[s]; continue; }
        int64_t n = batch * dims[s] * dims[s + 1];
        dec[s] = (float*)malloc((size_t)n * sizeof(float));
        if (!dec[s]) { rc = 3; goto done; }
        if (dtype == OR_TF32)
            for (int64_t i = 0; i < n; ++i) dec[s][i] = oracle_round_tf32(((const float*)B[s])[i]);
        else if (base.st[s] == OR_FP8)
            for (int64_t i = 0; i < n; ++i) dec[s][i] = oracle_fp8_to_f32(((const uint8_t*)B[s])[i]);
        else
            for (int64_t i = 0; i < n; ++i) dec[s][i] = dec16(base.st[s], ((const uint16_t*)B[s])[i]);
        base.Bf[s] = dec[s];
    }
    {
        job_t* jobs = (job_t*)calloc((size_t)nthreads, sizeof(job_t));
        pthread_t* th = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
        if (!jobs || !th) { free(jobs); free(th); rc = 3; goto done; }
        for (int t = 0; t < nthreads; ++t) {
            jobs[t] = base;
            jobs[t].r0 = nrows * t / nthreads;
            jobs[t].r1 = nrows * (t + 1) / nthreads;
        }
        int started = 0;
        for (int t = 1; t < nthreads; ++t) {
            if (pthread_create(&th[t], NULL, cascade_worker, &jobs[t]) != 0) break;
            started = t;
        }
        cascade_worker(&jobs[0]);
        for (int t = 1; t <= started; ++t) pthread_join(th[t], NULL);
        for (int t = started + 1; t < nthreads; ++t) cascade_worker(&jobs[t]);
        for (int t = 0; t < nthreads; ++t) if (jobs[t].err) rc = jobs[t].err;
        free(jobs); free(th);
    }
done:
    for (int s = 0; s < nstages; ++s) free(dec[s]);
    return rc;
}

int oracle_cascade(int dtype, int nstages, const int64_t* dims, int64_t batch, int64_t M,
                   const void* A, const void* const* B, const int64_t* rows, int64_t nrows,
                   void* D_out, int nthreads)
{
    return cascade_run(dtype, NULL, nstages, dims, batch, M, A, B, rows, nrows, D_out, nthreads);
}

/* types[0..nstages]: OR_F16 or OR_BF16 each; A in types[0], B_s in types[s],
   the result of GEMM s rounded into types[s + 1]; D in types[nstages] */
int oracle_cascade_typed(const int* types, int nstages, const int64_t* dims, int64_t batch, int64_t M,
                         const void* A, const void* const* B, const int64_t* rows, int64_t nrows,
                         void* D_out, int nthreads)
{
    if (!types) return 2;
    return cascade_run(types[0], types, nstages, dims, batch, M, A, B, rows, nrows, D_out, nthreads);
}
