// C-ABI entry points of libnvfp4 (declared and documented in include/nvfp4.h):
// argument validation on the host, then asynchronous launches on the caller's
// stream.  No allocation; the only state is a per-device cache of the compute
// unit count.
#include "../../include/mxfp4.h"
#include "../../include/nvfp4.h"
#include "nvfp4_launch.hpp"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

nvfp4_status check_tensor(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld) {
  if (x == nullptr) return NVFP4_EINVAL;
  if (dt != NVFP4_BF16 && dt != NVFP4_F32) return NVFP4_EINVAL;
  if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 16 != 0) return NVFP4_ESHAPE;
  if (ld < cols) return NVFP4_ESHAPE;
  if (rows > ((int64_t(1) << 32) - 1) / cols) return NVFP4_ESHAPE;  // element indices fit 32 bits
  if ((rows - 1) * ld + cols >= (int64_t(1) << 40)) return NVFP4_ESHAPE;
  const int64_t esize = dt == NVFP4_BF16 ? 2 : 4;
  if (!aligned16(x) || (ld * esize) % 16 != 0) return NVFP4_EALIGN;
  return NVFP4_OK;
}

nvfp4_status check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || M % 16 != 0 || N % 16 != 0 || K % 64 != 0) return NVFP4_ESHAPE;
  if (M >= (int64_t(1) << 31) || N >= (int64_t(1) << 31) || K >= (int64_t(1) << 31)) return NVFP4_ESHAPE;
  return NVFP4_OK;
}

nvfp4_status gemm_common(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                         const uint8_t* a_scales, const float* a_tensor_scale,
                         const uint8_t* b_codes, const uint8_t* b_scales, int32_t b_scale_rowdiv,
                         const float* b_tensor_scale, void* c, int c_bf16, int64_t ldc, float beta,
                         void* workspace, int64_t workspace_bytes, void* stream) {
  if (a_codes == nullptr || a_scales == nullptr || a_tensor_scale == nullptr ||
      b_codes == nullptr || b_scales == nullptr || b_tensor_scale == nullptr || c == nullptr)
    return NVFP4_EINVAL;
  if (b_scale_rowdiv != 1 && b_scale_rowdiv != 16) return NVFP4_EINVAL;
  if (beta != 0.0f && beta != 1.0f) return NVFP4_EINVAL;
  nvfp4_status st = check_gemm_shape(M, N, K);
  if (st != NVFP4_OK) return st;
  // the kernel addresses each operand's codes with 32-bit offsets
  if (M * (K / 2) >= (int64_t(1) << 32) || N * (K / 2) >= (int64_t(1) << 32)) return NVFP4_ESHAPE;
  if (ldc < N || workspace_bytes < 0) return NVFP4_ESHAPE;
  if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned4(a_scales) || !aligned4(b_scales) ||
      !aligned4(a_tensor_scale) || !aligned4(b_tensor_scale) || !aligned16(c) ||
      ldc % (c_bf16 ? 8 : 4) != 0 || !aligned16(workspace))
    return NVFP4_EALIGN;
  hipError_t e = nvfp4::launch_gemm(M, N, K, a_codes, a_scales, a_tensor_scale, b_codes, b_scales,
                                    b_scale_rowdiv, b_tensor_scale, c, c_bf16, ldc,
                                    beta == 1.0f ? 1 : 0, workspace,
                                    workspace == nullptr ? 0 : workspace_bytes,
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

}  // namespace

extern "C" {

nvfp4_status nvfp4_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x,
                            int layout, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                            uint8_t* codes_t, uint8_t* scales_t, float* tensor_scale, float* amax,
                            void* stream) {
  if (codes == nullptr || scales == nullptr || tensor_scale == nullptr || amax == nullptr)
    return NVFP4_EINVAL;
  if (layout != NVFP4_ROW_1D && layout != NVFP4_COL_1D && layout != NVFP4_TILE_2D) return NVFP4_EINVAL;
  if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_EINVAL;
  if (layout != NVFP4_TILE_2D && (codes_t != nullptr || scales_t != nullptr)) return NVFP4_EINVAL;
  if ((codes_t == nullptr) != (scales_t == nullptr)) return NVFP4_EINVAL;
  nvfp4_status st = check_tensor(x, dt, rows, cols, ld_x);
  if (st != NVFP4_OK) return st;
  if (!aligned16(codes) || !aligned16(scales) || (codes_t && !aligned16(codes_t)) ||
      (scales_t && !aligned16(scales_t)) || !aligned4(tensor_scale) || !aligned4(amax))
    return NVFP4_EALIGN;
  hipError_t e = nvfp4::launch_quantize(x, dt, rows, cols, ld_x, layout, rnd, seed, codes, scales,
                                        codes_t, scales_t, tensor_scale, amax,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status nvfp4_rht_quantize(const void* x, int dt, int64_t tokens, int64_t cols, int64_t ld_x,
                                uint32_t sign_mask, int rnd, uint64_t seed, uint8_t* codes,
                                uint8_t* scales, float* tensor_scale, float* amax, void* stream) {
  if (codes == nullptr || scales == nullptr || tensor_scale == nullptr || amax == nullptr)
    return NVFP4_EINVAL;
  if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_EINVAL;
  nvfp4_status st = check_tensor(x, dt, tokens, cols, ld_x);
  if (st != NVFP4_OK) return st;
  if (!aligned16(codes) || !aligned16(scales) || !aligned4(tensor_scale) || !aligned4(amax))
    return NVFP4_EALIGN;
  hipError_t e = nvfp4::launch_rht_quantize(x, dt, tokens, cols, ld_x, sign_mask, rnd, seed, codes,
                                            scales, tensor_scale, amax,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status nvfp4_quantize_row_rht(const void* x, int dt, int64_t tokens, int64_t cols,
                                    int64_t ld_x, int row_rnd, uint64_t row_seed,
                                    uint8_t* row_codes, uint8_t* row_scales,
                                    float* row_tensor_scale, float* row_amax, uint32_t sign_mask,
                                    int rht_rnd, uint64_t rht_seed, uint8_t* rht_codes,
                                    uint8_t* rht_scales, float* rht_tensor_scale, float* rht_amax,
                                    void* stream) {
  if (row_codes == nullptr || row_scales == nullptr || row_tensor_scale == nullptr ||
      row_amax == nullptr || rht_codes == nullptr || rht_scales == nullptr ||
      rht_tensor_scale == nullptr || rht_amax == nullptr)
    return NVFP4_EINVAL;
  if ((row_rnd != NVFP4_RNE && row_rnd != NVFP4_SR) || (rht_rnd != NVFP4_RNE && rht_rnd != NVFP4_SR))
    return NVFP4_EINVAL;
  nvfp4_status st = check_tensor(x, dt, tokens, cols, ld_x);
  if (st != NVFP4_OK) return st;
  if (!aligned16(row_codes) || !aligned16(row_scales) || !aligned16(rht_codes) ||
      !aligned16(rht_scales) || !aligned4(row_tensor_scale) || !aligned4(row_amax) ||
      !aligned4(rht_tensor_scale) || !aligned4(rht_amax))
    return NVFP4_EALIGN;
  hipError_t e = nvfp4::launch_quantize_row_rht(
      x, dt, tokens, cols, ld_x, row_rnd, row_seed, row_codes, row_scales, row_tensor_scale,
      row_amax, sign_mask, rht_rnd, rht_seed, rht_codes, rht_scales, rht_tensor_scale, rht_amax,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status nvfp4_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  if (bytes == nullptr) return NVFP4_EINVAL;
  nvfp4_status st = check_gemm_shape(M, N, K);
  if (st != NVFP4_OK) return st;
  *bytes = nvfp4::gemm_workspace_size(M, N, K);
  return NVFP4_OK;
}

nvfp4_status nvfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                        const uint8_t* a_scales, const float* a_tensor_scale,
                        const uint8_t* b_codes, const uint8_t* b_scales, int32_t b_scale_rowdiv,
                        const float* b_tensor_scale, float* c, int64_t ldc, float beta,
                        void* workspace, int64_t workspace_bytes, void* stream) {
  return gemm_common(M, N, K, a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_scale_rowdiv,
                     b_tensor_scale, c, 0, ldc, beta, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_gemm_noalloc(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                                const uint8_t* a_scales, const float* a_tensor_scale,
                                const uint8_t* b_codes, const uint8_t* b_scales,
                                int32_t b_scale_rowdiv, const float* b_tensor_scale, float* c,
                                int64_t ldc, float beta, void* stream) {
  if (a_codes == nullptr || a_scales == nullptr || a_tensor_scale == nullptr ||
      b_codes == nullptr || b_scales == nullptr || b_tensor_scale == nullptr || c == nullptr)
    return NVFP4_EINVAL;
  if (b_scale_rowdiv != 1 && b_scale_rowdiv != 16) return NVFP4_EINVAL;
  if (beta != 0.0f && beta != 1.0f) return NVFP4_EINVAL;
  nvfp4_status st = check_gemm_shape(M, N, K);
  if (st != NVFP4_OK) return st;
  if (M * (K / 2) >= (int64_t(1) << 32) || N * (K / 2) >= (int64_t(1) << 32) || ldc < N)
    return NVFP4_ESHAPE;
  if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned4(a_scales) || !aligned4(b_scales) ||
      !aligned4(a_tensor_scale) || !aligned4(b_tensor_scale) || !aligned16(c) || ldc % 4 != 0)
    return NVFP4_EALIGN;
  if (nvfp4::gemm_workspace_size(M, N, K) > nvfp4::static_workspace_bytes()) return NVFP4_ESCRATCH;
  hipError_t e = nvfp4::launch_gemm_static_ws(M, N, K, a_codes, a_scales, a_tensor_scale, b_codes,
                                              b_scales, b_scale_rowdiv, b_tensor_scale, c, ldc,
                                              beta == 1.0f ? 1 : 0, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status nvfp4_gemm_bf16(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                             const uint8_t* a_scales, const float* a_tensor_scale,
                             const uint8_t* b_codes, const uint8_t* b_scales,
                             int32_t b_scale_rowdiv, const float* b_tensor_scale, uint16_t* c,
                             int64_t ldc, float beta, void* workspace, int64_t workspace_bytes,
                             void* stream) {
  return gemm_common(M, N, K, a_codes, a_scales, a_tensor_scale, b_codes, b_scales, b_scale_rowdiv,
                     b_tensor_scale, c, 1, ldc, beta, workspace, workspace_bytes, stream);
}

nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales, int32_t scale_rowdiv,
                              const float* tensor_scale, int64_t rows, int64_t cols, int out_dt,
                              void* out, int64_t ld_out, void* stream) {
  if (codes == nullptr || scales == nullptr || tensor_scale == nullptr || out == nullptr)
    return NVFP4_EINVAL;
  if (scale_rowdiv != 1 && scale_rowdiv != 16) return NVFP4_EINVAL;
  if (out_dt != NVFP4_BF16 && out_dt != NVFP4_F32) return NVFP4_EINVAL;
  if (rows <= 0 || cols <= 0 || cols % 16 != 0 || rows % scale_rowdiv != 0 || ld_out < cols)
    return NVFP4_ESHAPE;
  if (rows > ((int64_t(1) << 32) - 1) / cols || (rows - 1) * ld_out + cols >= (int64_t(1) << 40))
    return NVFP4_ESHAPE;
  const int64_t esize = out_dt == NVFP4_BF16 ? 2 : 4;
  if (!aligned16(codes) || !aligned4(tensor_scale) || !aligned16(out) || (ld_out * esize) % 16 != 0)
    return NVFP4_EALIGN;
  hipError_t e = nvfp4::launch_dequantize(codes, scales, scale_rowdiv, tensor_scale, rows, cols, out,
                                          out_dt == NVFP4_BF16 ? 1 : 0, ld_out,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status mxfp4_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld_x,
                            int layout, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                            void* stream) {
  if (codes == nullptr || scales == nullptr) return NVFP4_EINVAL;
  if (layout != NVFP4_ROW_1D && layout != NVFP4_COL_1D) return NVFP4_EINVAL;
  if (rnd != NVFP4_RNE && rnd != NVFP4_SR) return NVFP4_EINVAL;
  nvfp4_status st = check_tensor(x, dt, rows, cols, ld_x);
  if (st != NVFP4_OK) return st;
  if ((layout == NVFP4_ROW_1D && cols % 32 != 0) || (layout == NVFP4_COL_1D && rows % 32 != 0))
    return NVFP4_ESHAPE;
  if (!aligned16(codes) || !aligned4(scales)) return NVFP4_EALIGN;
  hipError_t e = nvfp4::launch_mx_quantize(x, dt, rows, cols, ld_x, layout, rnd, seed, codes, scales,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status mxfp4_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                        const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                        float* c, int64_t ldc, float beta, void* workspace, int64_t workspace_bytes,
                        void* stream) {
  if (a_codes == nullptr || a_scales == nullptr || b_codes == nullptr || b_scales == nullptr ||
      c == nullptr)
    return NVFP4_EINVAL;
  if (beta != 0.0f && beta != 1.0f) return NVFP4_EINVAL;
  nvfp4_status st = check_gemm_shape(M, N, K);
  if (st != NVFP4_OK) return st;
  if (K % 128 != 0 || ldc < N || workspace_bytes < 0) return NVFP4_ESHAPE;
  if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned4(a_scales) || !aligned4(b_scales) ||
      !aligned16(c) || ldc % 4 != 0 || !aligned16(workspace))
    return NVFP4_EALIGN;
  hipError_t e = nvfp4::launch_mx_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales, c, ldc,
                                       beta == 1.0f ? 1 : 0, workspace,
                                       workspace == nullptr ? 0 : workspace_bytes,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status nvfp4_set_quantize_passes(int passes) {
  if (passes != 0 && passes != 2) return NVFP4_EINVAL;
  return nvfp4::set_quantize_passes(passes) == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status nvfp4_set_sync_spin_limit(int64_t polls) {
  if (polls < 0) return NVFP4_EINVAL;
  return nvfp4::set_sync_spin_limit((uint64_t)polls) == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

nvfp4_status nvfp4_single_pass_stats(int64_t* launches, int64_t* give_ups) {
  if (launches == nullptr || give_ups == nullptr) return NVFP4_EINVAL;
  return nvfp4::single_pass_stats(launches, give_ups) == hipSuccess ? NVFP4_OK : NVFP4_EHIP;
}

const char* nvfp4_status_str(int status) {
  switch (status) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_EINVAL: return "NVFP4_EINVAL: null pointer or invalid argument value";
    case NVFP4_ESHAPE: return "NVFP4_ESHAPE: unsupported shape";
    case NVFP4_EALIGN: return "NVFP4_EALIGN: misaligned pointer or leading dimension";
    case NVFP4_EHIP: return "NVFP4_EHIP: HIP launch failed";
    case NVFP4_ESCRATCH:
      return "NVFP4_ESCRATCH: the problem needs more split workspace than the static scratch holds";
    default: return "unknown nvfp4 status";
  }
}

}  // extern "C"
