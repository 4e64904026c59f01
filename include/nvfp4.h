/*
 * libnvfp4 -- NVFP4 quantize-and-contract for one linear layer on MI355X (gfx950).
 *
 * The method ("Pretraining Large Language Models with NVFP4", gist.science
 * summary, section "Resumo tecnico", part 2 "Metodologia Proposta"):
 *   - NVFP4 stores FP4 (E2M1) values in blocks of 16 with one FP8 E4M3 scale
 *     per block and one FP32 scale per tensor (bullets "Bloco Menor",
 *     "Fatores de Escala Precisos", "Escala em Dois Niveis");
 *   - weights are scaled per 16x16 tile so forward and backward use the same
 *     quantized weight (technique 3, "Escala Bidimensional (2D) para Pesos");
 *   - the Wgrad inputs go through a 16x16 random Hadamard transform
 *     (technique 2; the 16x16 size is stated in "NVIDIA cria metodo para
 *     treinar redes neurais com precisao de 4 bits", section "Como funciona");
 *   - gradients use stochastic rounding, everything else round-to-nearest-even
 *     (technique 4, "Arredondamento Estocastico").
 * Arithmetic details the pages leave open are fixed as follows (IEEE binary32,
 * round-to-nearest-even, in this order):
 *   amax_t = max |y| over the tensor (y = x, or the RHT output)
 *   S_enc  = amax_t > 0 ? min(2688 / amax_t, FLT_MAX) : 1;  tensor_scale = 1 / S_enc
 *   e_b    = E4M3 nearest-even, saturating at 448, of (amax_b / 6) * S_enc
 *   r_b    = e_b == 0 ? 0 : min(S_enc / dec(e_b), FLT_MAX);   v = y * r_b
 *   code   = sign(y) << 3 | E2M1 index of |v|: RNE (ties to even index,
 *            saturating at 6) or SR: with a = min(|v|, 6) between the E2M1
 *            magnitudes lo <= a < hi and frac = (a - lo) / (hi - lo) taken
 *            exactly, round up iff r16 < frac * 65536, so P(up) =
 *            ceil(frac * 65536) / 65536 (technique 4, "Arredondamento
 *            Estocastico": rounding up with probability given by the distance
 *            keeps the expected value).  r16 = 16 bits of the pcg hash of
 *            Jarzynski & Olano, JCGT 2020: key = pcg(lo32(seed) ^
 *            pcg(hi32(seed))), w = pcg(key ^ (i >> 1)), r16 = the low half of w
 *            for even i and the high half for odd i, i the element's index in
 *            the output code array.
 *   Dequantized value = e2m1(code) * dec(e_b) * tensor_scale.
 *
 * Packing: two codes per byte, the even element in the low nibble.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates and frees nothing and is reentrant; calls on different streams
 *     may overlap (but not while sharing a GEMM workspace).  Its state is a
 *     per-device cache of the compute-unit count and occupancy, and two static
 *     device arrays per device: the exchange slots of the quantize calls' amax
 *     reductions (64 slots of 18.25 KiB, one per stream in use, with a host
 *     epoch counter each) and the split workspace of nvfp4_gemm_noalloc
 *     (64 MiB).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued asynchronously on it; results are visible after the
 *     caller synchronizes that stream.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     return NVFP4_EINVAL / NVFP4_ESHAPE / NVFP4_EALIGN; NVFP4_EHIP means a
 *     launch failed.  Faults during execution surface at the caller's
 *     synchronization.
 *   - Inputs must be finite; codes for NaN/Inf inputs are unspecified.
 *   - Tensor element counts must stay below 2^32.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_EINVAL = 1, /* null pointer, unknown enum value, bad rowdiv/beta */
    NVFP4_ESHAPE = 2, /* dimension not a multiple of 16 (quantize) or of the GEMM tile */
    NVFP4_EALIGN = 3, /* pointer or leading dimension not 16-byte aligned */
    NVFP4_EHIP = 4,   /* a HIP launch failed */
    NVFP4_ESCRATCH = 5 /* nvfp4_gemm_noalloc: more split workspace than its static scratch */
} nvfp4_status;

typedef enum { NVFP4_BF16 = 0, NVFP4_F32 = 1 } nvfp4_dtype;
typedef enum { NVFP4_RNE = 0, NVFP4_SR = 1 } nvfp4_rounding;
typedef enum { NVFP4_ROW_1D = 0, NVFP4_COL_1D = 1, NVFP4_TILE_2D = 2 } nvfp4_layout;

/*
 * Arguments that take one of these enums (dt, layout, rnd, out_dt, and the
 * status of nvfp4_status_str) are declared `int`: the width is fixed on every
 * C and C++ compiler and foreign-function binding, and a value outside the
 * enum reaches the library, which answers NVFP4_EINVAL (nvfp4_status_str:
 * "unknown nvfp4 status") instead of depending on how the caller's language
 * converts it.
 */

/*
 * nvfp4_quantize -- amax, two-level scales and E2M1 cast of one tensor.
 * ("Formato NVFP4" and techniques 3-4 of "Metodologia Proposta".)
 *
 *   x        [rows x cols] row-major, element type `dt`, leading dimension ld_x
 *            elements (ld_x >= cols; ld_x * elem_size a multiple of 16 bytes).
 *   layout   NVFP4_ROW_1D : blocks of 16 along a row (activations X for Fprop,
 *                           gradients dY for Dgrad).
 *                codes  [rows][cols/2], scales [rows][cols/16]
 *            NVFP4_COL_1D : blocks of 16 along a column, written transposed
 *                           (token-contiguous Wgrad operand without the RHT).
 *                codes  [cols][rows/2], scales [cols][rows/16]
 *            NVFP4_TILE_2D: one scale per 16x16 tile (weights).
 *                codes  [rows][cols/2], scales [rows/16][cols/16]
 *                codes_t [cols][rows/2], scales_t [cols/16][rows/16]: the SAME
 *                quantized values transposed (the Dgrad operand); both may be
 *                NULL to skip them.  Must be NULL for the 1D layouts.
 *   rnd, seed  NVFP4_RNE, or NVFP4_SR with the 64-bit hash seed.  The SR index
 *              of an element is its position in `codes` (r*cols + c for
 *              ROW_1D and TILE_2D, c*rows + r for COL_1D).
 *   tensor_scale, amax  one float each (device): outputs 1/S_enc and amax_t.
 *   rows, cols must be positive multiples of 16; all pointers 16-byte aligned
 *   except tensor_scale / amax (4-byte).
 *   Passes: the tensor amax is needed before any element is encoded ("Escala
 *   em Dois Niveis").  A contiguous (ld_x == cols) ROW_1D tensor that fits in
 *   the registers of one resident grid (on a 256-CU MI355X up to 84 MB of
 *   bf16, e.g. 8192 x 5120, or 42 MB of FP32) is read ONCE: a grid no larger
 *   than what fits on the device at once keeps it on chip while its
 *   workgroups exchange the amax through a per-(device, stream) slot of
 *   library-owned device memory, then encodes it.  The wait is bounded: a
 *   workgroup that waits too long (its grid partly displaced by other
 *   streams' kernels) leaves its blocks to the workgroup that publishes the
 *   amax (the last to arrive), which encodes them from memory after its own,
 *   so the outputs are always complete.
 *   Everything else, and any call on a stream under graph capture, takes two
 *   passes (amax, then cast).  Both give identical outputs.  Calls on one
 *   stream never share a slot with another stream's calls (64 slots per
 *   device; further streams take two passes).
 */
nvfp4_status nvfp4_quantize(const void *x, int dt, int64_t rows, int64_t cols, int64_t ld_x,
                            int layout, int rnd, uint64_t seed, uint8_t *codes, uint8_t *scales,
                            uint8_t *codes_t, uint8_t *scales_t, float *tensor_scale,
                            float *amax, void *stream);

/*
 * nvfp4_rht_quantize -- random Hadamard transform along tokens, then 1D
 * column quantization of a Wgrad operand (technique 2 of "Metodologia
 * Proposta"; 16x16 per "Como funciona").
 *
 *   x [tokens x cols] row-major (ld_x elements).  For every column c and every
 *   group g of 16 consecutive tokens: u_j = x[16g + j][c], negated where bit j
 *   of sign_mask is set; radix-2 Walsh-Hadamard butterflies with strides
 *   1, 2, 4, 8 ((a, b) -> (a + b, a - b)); y_j = 0.25 * u_j.  That is
 *   y = (1/4) H16 diag(d) x, orthonormal, so the same sign_mask on dY and X
 *   cancels in dW = dY^T X.  amax_t is taken over y; each group is one block.
 *   codes [cols][tokens/2], scales [cols][tokens/16] (token-contiguous).
 *   SR index of an element: c*tokens + t.
 *   tokens, cols positive multiples of 16; sign_mask uses its low 16 bits.
 */
nvfp4_status nvfp4_rht_quantize(const void *x, int dt, int64_t tokens, int64_t cols, int64_t ld_x,
                                uint32_t sign_mask, int rnd, uint64_t seed, uint8_t *codes,
                                uint8_t *scales, float *tensor_scale, float *amax, void *stream);

/*
 * nvfp4_quantize_row_rht -- both quantizations a tensor needs in one linear
 * layer: the row-1D one (X for Fprop, dY for Dgrad) and the RHT column one
 * (X, dY for Wgrad).  Its outputs are exactly those of
 *   nvfp4_quantize(x, dt, tokens, cols, ld_x, NVFP4_ROW_1D, row_rnd, row_seed,
 *                  row_codes, row_scales, NULL, NULL, row_tensor_scale, row_amax)
 *   nvfp4_rht_quantize(x, dt, tokens, cols, ld_x, sign_mask, rht_rnd, rht_seed,
 *                      rht_codes, rht_scales, rht_tensor_scale, rht_amax)
 * (same layouts, SR indices and errors), but both tensor amaxes (of x and of
 * its RHT) come from ONE read of x, saving a full pass over the tensor.
 * With RNE on both copies, a bf16 tensor whose 256 x 128 tiles fit in the
 * registers of one resident grid (two per workgroup: up to 8192 x 6144 on
 * a 256-CU MI355X) is read only once in all: one launch takes both maxima,
 * exchanges them between its workgroups and encodes from registers (the
 * single-pass path below; same outputs).  The two output sets must not
 * overlap.
 */
nvfp4_status nvfp4_quantize_row_rht(const void *x, int dt, int64_t tokens, int64_t cols,
                                    int64_t ld_x, int row_rnd, uint64_t row_seed,
                                    uint8_t *row_codes, uint8_t *row_scales,
                                    float *row_tensor_scale, float *row_amax, uint32_t sign_mask,
                                    int rht_rnd, uint64_t rht_seed, uint8_t *rht_codes,
                                    uint8_t *rht_scales, float *rht_tensor_scale, float *rht_amax,
                                    void *stream);

/*
 * nvfp4_gemm -- block-scaled NVFP4 contraction with FP32 accumulation
 * (the NVFP4 GEMMs of "Suporte de Hardware", part 3 of the same page).
 *
 *   C[m][n] = beta * C[m][n]
 *           + a_ts * b_ts * sum_k (e2m1(A[m][k]) * dec(sA[m][k/16]))
 *                                * (e2m1(B[n][k]) * dec(sB[n/b_scale_rowdiv][k/16]))
 *   Both operands are K-contiguous ("NT"):
 *     a_codes [M][K/2], a_scales [M][K/16]                       (1D scales)
 *     b_codes [N][K/2], b_scales [N/b_scale_rowdiv][K/16]       (rowdiv 1: 1D,
 *                                                               16: 2D tile grid)
 *     a_tensor_scale, b_tensor_scale: one device float each (tensor_scale
 *     outputs of the quantize calls).
 *     c [M][ldc] FP32, ldc >= N.  beta must be 0 (overwrite) or 1 (accumulate).
 *   Fprop Y = X W^T : A = X row-1D, B = W tile-2D codes/scales (rowdiv 16).
 *   Dgrad dX = dY W : A = dY row-1D, B = W tile-2D codes_t/scales_t (rowdiv 16).
 *   Wgrad dW = dY^T X: A = RHT(dY) column-1D, B = RHT(X) column-1D (rowdiv 1),
 *                      K = tokens.
 *   M and N must be positive multiples of 16, K a positive multiple of 64 (all
 *   below 2^31), and each operand's code array below 4 GiB (M*K/2 and N*K/2 <
 *   2^32); ldc >= N and a multiple of 4; c 16-byte aligned.
 *   Products e2m1 * E4M3 are exact in FP16, so the kernel dequantizes the
 *   block-scaled operands exactly and contracts them on FP16 matrix cores with
 *   FP32 accumulation; the two tensor scales are applied in the epilogue.
 *   workspace, workspace_bytes: optional device scratch (16-byte aligned) of at
 *   least nvfp4_gemm_workspace_size() bytes.  With it, the output tiles of an
 *   incomplete last round over the compute units are split along K and their
 *   FP32 partial sums are added in a fixed order by a second kernel on the
 *   same stream (deterministic: the result depends only on the shape and the
 *   inputs).  NULL, or fewer bytes than needed, runs without the split (same
 *   result up to FP32 summation order).  The workspace is in use until the
 *   call's work on `stream` completes.
 *   The same call without the workspace pair, (M, N, K, a_codes, a_scales,
 *   a_tensor_scale, b_codes, b_scales, b_scale_rowdiv, b_tensor_scale, c,
 *   ldc, beta, stream), is nvfp4_gemm_noalloc below; it splits into the
 *   library's own static scratch and gives, bit for bit, the result of this
 *   call with a large enough workspace.
 */
nvfp4_status nvfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t *a_codes,
                        const uint8_t *a_scales, const float *a_tensor_scale,
                        const uint8_t *b_codes, const uint8_t *b_scales, int32_t b_scale_rowdiv,
                        const float *b_tensor_scale, float *c, int64_t ldc, float beta,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * nvfp4_gemm_noalloc -- nvfp4_gemm for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace pair, the same
 * FP32 result as nvfp4_gemm given a workspace of nvfp4_gemm_workspace_size()
 * bytes (bit for bit: same kernels, same split of the last round of tiles).
 * The split partials live in a file-scope static device array of 64 MiB, one
 * per device, held until the process ends (256 KiB per compute unit of a
 * 256-CU MI355X, the most the split plan uses there).  It allocates nothing:
 * no hipMalloc, hipFree or allocating library call.  Every call on a device
 * shares that device's array, so calls that overlap on one device (different
 * streams, or graph replays in flight together) race; calls on one stream are
 * safe.  A shape whose split would need more than the static array (possible
 * only on a device with more than 256 compute units) returns NVFP4_ESCRATCH
 * before anything is enqueued.  Other errors as for nvfp4_gemm.
 */
nvfp4_status nvfp4_gemm_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t *a_codes,
                                const uint8_t *a_scales, const float *a_tensor_scale,
                                const uint8_t *b_codes, const uint8_t *b_scales,
                                int32_t b_scale_rowdiv, const float *b_tensor_scale, float *c,
                                int64_t ldc, float beta, void *stream);

/*
 * nvfp4_gemm_bf16 -- nvfp4_gemm with a BF16 output: every argument as for
 * nvfp4_gemm except c, which holds BF16 bit patterns [M][ldc] (ldc a multiple
 * of 8, c 16-byte aligned).  Each output is computed in FP32 exactly as by
 * nvfp4_gemm (alpha * accumulated sum, plus the BF16 value already in c
 * widened to FP32 when beta = 1) and rounded to BF16 once, to nearest even.
 * The pages' recipe keeps the rest of the model in BF16 (same page, part 2,
 * technique 1, the layers left in BF16), so a linear layer's result returns
 * to BF16; the rounding taken is the plain nearest-even one of the FP32
 * result.
 */
nvfp4_status nvfp4_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint8_t *a_codes,
                             const uint8_t *a_scales, const float *a_tensor_scale,
                             const uint8_t *b_codes, const uint8_t *b_scales,
                             int32_t b_scale_rowdiv, const float *b_tensor_scale, uint16_t *c,
                             int64_t ldc, float beta, void *workspace, int64_t workspace_bytes,
                             void *stream);

/*
 * nvfp4_dequantize -- NVFP4 codes back to FP32 or BF16 (the value definition
 * of "Formato NVFP4", part 2 of the same page: E2M1 element x E4M3 block scale
 * x FP32 tensor scale).
 *
 *   out[r][c] = RN32( e2m1(code[r][c]) * dec(scales[r / scale_rowdiv][c / 16])
 *                     * tensor_scale[0] )
 *   rows x cols is the shape of the code array as stored: codes [rows][cols/2]
 *   (the even element in the low nibble); scales [rows][cols/16] with
 *   scale_rowdiv 1 (row-1D, column-1D and RHT outputs, read in their stored,
 *   transposed orientation) or [rows/16][cols/16] with scale_rowdiv 16 (the
 *   2D tile grid; codes_t / scales_t of a 2D quantization dequantize the same
 *   way).  e2m1 * dec is exact in FP32, so the only rounding is the multiply
 *   by the tensor scale (RN32, nearest even); out_dt NVFP4_BF16 rounds that
 *   FP32 value to BF16, nearest even.  out [rows][ld_out] of out_dt, 16-byte
 *   aligned rows (ld_out * element size a multiple of 16); ld_out >= cols.
 *   cols a positive multiple of 16, rows a positive multiple of scale_rowdiv,
 *   rows * cols < 2^32.  Scale bytes must be finite E4M3 codes (0x00..0x7E,
 *   what the quantize calls produce); codes 0x7F/0xFF give unspecified values.
 */
nvfp4_status nvfp4_dequantize(const uint8_t *codes, const uint8_t *scales, int32_t scale_rowdiv,
                              const float *tensor_scale, int64_t rows, int64_t cols, int out_dt,
                              void *out, int64_t ld_out, void *stream);

/*
 * nvfp4_gemm_workspace_size -- bytes of workspace nvfp4_gemm uses for an
 * M x N x K problem on the CURRENT device (0 when that shape needs none; at
 * most 256 KiB per compute unit).  Shape rules and errors as for nvfp4_gemm;
 * `bytes` must not be NULL.
 */
nvfp4_status nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t *bytes);

/*
 * Controls and counters of the single-pass quantize paths (nvfp4_quantize
 * ROW_1D, nvfp4_quantize_row_rht on bf16).  Process-wide settings, safe to
 * call from any thread.
 *   nvfp4_set_quantize_passes(passes): 0 (default) picks the single pass where
 *     it applies; 2 always takes the two-pass path.  Other values: EINVAL.
 *   nvfp4_set_sync_spin_limit(polls): how many times a workgroup polls the
 *     device-wide exchange (about 1 us each) before it gives up and leaves its
 *     blocks to the last workgroup (default 2^14, far beyond the wait of a
 *     resident grid).  Giving up changes only the speed, never the result;
 *     tests use it to force that path from the host.  polls >= 0.
 *   nvfp4_single_pass_stats(launches, give_ups): on the CURRENT device since
 *     the library was loaded, the number of single-pass launches enqueued and
 *     of their workgroups that gave up waiting (a synchronous device read;
 *     call after synchronizing the streams in question).  Both pointers are
 *     host pointers.
 */
nvfp4_status nvfp4_set_quantize_passes(int passes);
nvfp4_status nvfp4_set_sync_spin_limit(int64_t polls);
nvfp4_status nvfp4_single_pass_stats(int64_t *launches, int64_t *give_ups);

/* Static, human-readable name of a status code. */
const char *nvfp4_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
