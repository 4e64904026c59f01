/*
 * libnvfp4, MXFP4 entry points -- the comparison format, on gfx950's native
 * block-scaled FP4 matrix instruction.
 *
 * MXFP4 ("Pretraining Large Language Models with NVFP4", gist.science
 * summary, section "Resumo tecnico", part 1 "Limitacoes de Formatos
 * Existentes" and part 2 "Fatores de Escala Precisos"): FP4 (E2M1) values in
 * blocks of 32 with one power-of-two UE8M0 scale per block, no tensor scale.
 * Conversion per the OCP Microscaling Formats (MX) v1.0 specification:
 *   e    = floor(log2(max |x| over the block)) - 2, clamped to [-127, 127]
 *          (2 is the largest E2M1 exponent; an all-zero block takes -127)
 *   code = E2M1 of x * 2^-e: nearest-even (saturating at 6) or stochastic
 *          rounding with the same pcg bits, keyed by the element's index in
 *          the output code array, as nvfp4_quantize
 *   scale byte = e + 127.   Dequantized value = e2m1(code) * 2^(scale - 127).
 * Packing: two codes per byte, the even element in the low nibble.
 *
 * Status codes, dtype / rounding / layout enums, pointer ownership, stream and
 * error conventions: as in nvfp4.h.
 */
#ifndef MXFP4_H
#define MXFP4_H

#include "nvfp4.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * mxfp4_quantize -- one pass over x (each block's scale depends only on the
 * block).
 *   x      [rows x cols] row-major, element type `dt`, leading dimension ld_x
 *          (ld_x >= cols, ld_x * elem_size a multiple of 16 bytes).
 *   layout NVFP4_ROW_1D: blocks of 32 along a row;
 *                        codes [rows][cols/2], scales [rows][cols/32];
 *                        cols a multiple of 32, rows of 16.
 *          NVFP4_COL_1D: blocks of 32 along a column, written transposed;
 *                        codes [cols][rows/2], scales [cols][rows/32];
 *                        rows a multiple of 32, cols of 16.
 *   rnd, seed  NVFP4_RNE, or NVFP4_SR with the 64-bit hash seed.
 *   codes 16-byte aligned, scales 4-byte aligned.
 */
nvfp4_status mxfp4_quantize(const void *x, int dt, int64_t rows, int64_t cols, int64_t ld_x,
                            int layout, int rnd, uint64_t seed, uint8_t *codes, uint8_t *scales,
                            void *stream);

/*
 * mxfp4_gemm -- C[m][n] = beta * C[m][n]
 *               + sum_k (e2m1(A[m][k]) 2^(sA[m][k/32]-127)) (e2m1(B[n][k]) 2^(sB[n][k/32]-127))
 * Both operands K-contiguous ("NT"): a_codes [M][K/2], a_scales [M][K/32],
 * b_codes [N][K/2], b_scales [N][K/32].  The products are exact and summed in
 * FP32 by the block-scaled FP4 matrix instruction.
 * M, N positive multiples of 16, K a positive multiple of 128 (below 2^31);
 * ldc >= N and a multiple of 4; codes and c 16-byte aligned, scales 4-byte
 * aligned; beta 0 or 1.  workspace / workspace_bytes: as for nvfp4_gemm (the
 * size nvfp4_gemm_workspace_size reports for the same M, N, K; NULL runs
 * without the tail split).
 */
nvfp4_status mxfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *a_codes,
                        const uint8_t *a_scales, const uint8_t *b_codes, const uint8_t *b_scales,
                        float *c, int64_t ldc, float beta, void *workspace, int64_t workspace_bytes,
                        void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H */
