/* Drives the C oracle (encoders, decoders, one stage, cascades of every type,
 * several threads) on small random inputs, for a build with AddressSanitizer
 * and UndefinedBehaviorSanitizer.  The values are checked by the Python pins;
 * here only memory and undefined-behaviour errors count.  Exit status 0. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_f32_to_f16(float x);
float oracle_f16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float x);
float oracle_bf16_to_f32(uint16_t h);
float oracle_round_tf32(float x);
float oracle_fp8_to_f32(uint8_t c);
uint8_t oracle_f32_to_fp8(float x);
int oracle_gemm_acc(int dtype, int64_t M, int64_t K, int64_t N, const void* X, const void* B, void* acc_out);
int oracle_cascade(int dtype, int nstages, const int64_t* dims, int64_t batch, int64_t M, const void* A,
                   const void* const* B, const int64_t* rows, int64_t nrows, void* D_out, int nthreads);
int oracle_cascade_typed(const int* types, int nstages, const int64_t* dims, int64_t batch, int64_t M,
                         const void* A, const void* const* B, const int64_t* rows, int64_t nrows, void* D_out,
                         int nthreads);

static uint32_t rng = 0x12345678u;
static float frand(void) { rng = rng * 1664525u + 1013904223u; return (float)((rng >> 8) * (1.0 / 16777216.0)) * 2.f - 1.f; }

int main(void) {
    /* every 16-bit code through both decoders and back; a sweep of fp32 patterns */
    unsigned sum = 0;
    for (uint32_t h = 0; h < 65536; ++h) {
        sum += oracle_f32_to_f16(oracle_f16_to_f32((uint16_t)h));
        sum += oracle_f32_to_bf16(oracle_bf16_to_f32((uint16_t)h));
    }
    for (uint64_t u = 0; u < ((uint64_t)1 << 32); u += 65521) {
        float x;
        uint32_t v = (uint32_t)u;
        memcpy(&x, &v, 4);
        sum += oracle_f32_to_f16(x) + oracle_f32_to_bf16(x) + oracle_f32_to_fp8(x);
        float t = oracle_round_tf32(x);
        sum += (unsigned)(t == t);
    }
    for (int c = 0; c < 256; ++c) sum += (unsigned)(oracle_fp8_to_f32((uint8_t)c) == 0.f);

    /* cascades: types 0 f16, 1 bf16, 2 f64, 3 tf32; 1-3 stages, odd sizes, 1 and 3 threads */
    const int64_t dims[4] = {7, 5, 9, 3};
    const int64_t batch = 2, M = 11;
    for (int dt = 0; dt < 4; ++dt)
        for (int nst = 1; nst <= 3; ++nst)
            for (int th = 1; th <= 3; th += 2) {
                size_t esz = dt == 2 ? 8 : (dt == 3 ? 4 : 2);
                void* A = malloc((size_t)(batch * M * dims[0]) * esz);
                void* Bs[3];
                for (int s = 0; s < nst; ++s) Bs[s] = malloc((size_t)(batch * dims[s] * dims[s + 1]) * esz);
                void* D = malloc((size_t)(batch * M * dims[nst]) * esz);
                void* bufs[4] = {A, Bs[0], nst > 1 ? Bs[1] : NULL, nst > 2 ? Bs[2] : NULL};
                int64_t counts[4] = {batch * M * dims[0], batch * dims[0] * dims[1], batch * dims[1] * dims[2],
                                     batch * dims[2] * dims[3]};
                for (int i = 0; i <= nst; ++i)
                    for (int64_t j = 0; j < counts[i]; ++j) {
                        float f = frand();
                        if (dt == 2) ((double*)bufs[i])[j] = f;
                        else if (dt == 3) ((float*)bufs[i])[j] = f;
                        else ((uint16_t*)bufs[i])[j] = dt == 0 ? oracle_f32_to_f16(f) : oracle_f32_to_bf16(f);
                    }
                if (oracle_cascade(dt, nst, dims, batch, M, A, (const void* const*)Bs, NULL, 0, D, th)) return 2;
                const int64_t rows[3] = {0, 12, 21};
                if (oracle_cascade(dt, nst, dims, batch, M, A, (const void* const*)Bs, rows, 3, D, th)) return 3;
                if (dt < 2) {
                    int types[4] = {dt, 1 - dt, dt, 1 - dt};
                    if (oracle_cascade_typed(types, nst, dims, batch, M, A, (const void* const*)Bs, NULL, 0, D, th))
                        return 4;
                }
                float acc[11 * 5];
                double accd[11 * 5];
                if (oracle_gemm_acc(dt, M, dims[0], dims[1], A, Bs[0], dt == 2 ? (void*)accd : (void*)acc)) return 5;
                free(A);
                for (int s = 0; s < nst; ++s) free(Bs[s]);
                free(D);
            }
    printf("oracle driver: checksum %u\n", sum);
    return 0;
}
