// NVFP4 -> FP32 / BF16 dequantization for gfx950.
//
// Method: "Pretraining Large Language Models with NVFP4" (gist.science
// summary), Resumo tecnico, 2. Metodologia Proposta, "Formato NVFP4": a value
// is its E2M1 element times its block's E4M3 scale times the tensor's FP32
// scale.  e2m1(q) * dec(e) has at most 6 significant bits, so it is exact in
// FP32, and the multiply by the tensor scale rounds once; BF16 output rounds
// that FP32 value to nearest even.
//
// HBM-bound (0.5625 B read, 4 or 2 B written per element): each thread
// expands one 16-element block (8 code bytes, one scale byte) to 16 outputs,
// consecutive threads taking consecutive blocks of a row, so code loads and
// output stores are contiguous across a wave.
#include <algorithm>

#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

namespace {

// E2M1 codes of one dword (8 elements, element 0 in the low nibble) -> FP32.
// (scale 1.0: the conversion is exact)
__device__ __forceinline__ void e2m1x8(uint32_t w, float* v) {
  const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  v[0] = f0[0]; v[1] = f0[1]; v[2] = f1[0]; v[3] = f1[1];
  v[4] = f2[0]; v[5] = f2[1]; v[6] = f3[0]; v[7] = f3[1];
}

template <typename OutT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes,
                                                 const uint8_t* __restrict__ scales, int rowdiv,
                                                 const float* __restrict__ ts, int64_t rows,
                                                 int64_t cols, OutT* __restrict__ out, int64_t ld) {
  const int64_t bpr = cols / 16;  // blocks per row
  const int64_t nblk = rows * bpr;
  const float s_t = ts[0];
  for (int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x; b < nblk; b += (int64_t)gridDim.x * 256) {
    const int64_t r = b / bpr, cb = b - r * bpr;
    const uint2 q = *reinterpret_cast<const uint2*>(codes + r * (cols / 2) + cb * 8);
    const float d = e4m3_decode(scales[(r / rowdiv) * bpr + cb]);
    float v[16];
    e2m1x8(q.x, v);
    e2m1x8(q.y, v + 8);
#pragma unroll
    for (int j = 0; j < 16; j++) v[j] = (v[j] * d) * s_t;
    OutT* o = out + r * ld + cb * 16;
    if constexpr (sizeof(OutT) == 4) {
      float4* o4 = reinterpret_cast<float4*>(o);
#pragma unroll
      for (int k = 0; k < 4; k++) o4[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
    } else {
      uint32_t p[8];
#pragma unroll
      for (int k = 0; k < 8; k++) p[k] = bf16_rne(v[2 * k]) | (bf16_rne(v[2 * k + 1]) << 16);
      uint4* o4 = reinterpret_cast<uint4*>(o);
      o4[0] = make_uint4(p[0], p[1], p[2], p[3]);
      o4[1] = make_uint4(p[4], p[5], p[6], p[7]);
    }
  }
}

}  // namespace

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int scale_rowdiv,
                             const float* tensor_scale, int64_t rows, int64_t cols, void* out,
                             int out_bf16, int64_t ld_out, hipStream_t s) {
  const int64_t nblk = rows * (cols / 16);
  const unsigned grid = (unsigned)std::min<int64_t>((nblk + 255) / 256, 4096);
  if (out_bf16)
    k_dequant<uint16_t><<<grid, 256, 0, s>>>(codes, scales, scale_rowdiv, tensor_scale, rows, cols,
                                             static_cast<uint16_t*>(out), ld_out);
  else
    k_dequant<float><<<grid, 256, 0, s>>>(codes, scales, scale_rowdiv, tensor_scale, rows, cols,
                                          static_cast<float*>(out), ld_out);
  return hipGetLastError();
}

}  // namespace nvfp4
