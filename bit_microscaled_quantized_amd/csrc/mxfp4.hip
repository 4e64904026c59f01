// MXFP4 quantization kernels for gfx950 (the comparison format).
//
// MXFP4 ("Pretraining Large Language Models with NVFP4", gist.science summary,
// Resumo tecnico, parts 1 and 2): FP4 E2M1 values in blocks of 32 with one
// power-of-two (UE8M0) scale per block and no tensor scale.  Conversion per
// the OCP MX v1.0 specification: shared exponent e = floor(log2(max |V|)) - 2
// (2 = the largest E2M1 exponent), clamped to [-127, 127]; elements V / 2^e
// rounded to E2M1 (nearest-even, or stochastic with the same pcg bits as the
// NVFP4 path) and clamped to +-6.
//
// Because a block's scale depends on that block alone, quantization is ONE
// pass: read 32 elements, write 16 code bytes and one scale byte -- bound by
// HBM bandwidth.  For the maximum's biased FP32 exponent field E (0 for zero
// and subnormal maxima), e = max(E - 129, -127) and the E8M0 code is e + 127;
// V / 2^e is one FP32 multiply by the exact power of two 2^-e.
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

namespace {

// e + 127 and 2^-e for a block maximum (amax >= 0, finite).
__device__ __forceinline__ void mx_scale(float amax, uint32_t& code, float& mul) {
  const int E = (int)(__float_as_uint(amax) >> 23);
  const int e = max(E - 129, -127);
  code = (uint32_t)(e + 127);
  mul = __uint_as_float((uint32_t)(127 - e) << 23);
}

// 32 scaled values -> 16 code bytes (element 0 in the low nibble of x);
// SR bits for output elements 2 pair0 .. 2 pair0 + 31 (pair0 a multiple of 16).
template <int RND>
__device__ __forceinline__ uint4 mx_encode32(const float* v, uint32_t key, uint32_t pair0) {
  if constexpr (RND == 0) {
    return make_uint4(pack8_rne(v), pack8_rne(v + 8), pack8_rne(v + 16), pack8_rne(v + 24));
  } else {
    uint32_t w[4];
#pragma unroll
    for (int half = 0; half < 2; half++) {
      uint32_t h[8];
      pcg8(key, pair0 + 8 * half, h);
      w[2 * half] = sr_pack8(v + 16 * half, h);
      w[2 * half + 1] = sr_pack8(v + 16 * half + 8, h + 4);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

template <typename T>
__device__ __forceinline__ void load32(const T* p, float* v);

template <>
__device__ __forceinline__ void load32<uint16_t>(const uint16_t* p, float* v) {
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint4 w = reinterpret_cast<const uint4*>(p)[q];
    v[8 * q + 0] = bf16lo(w.x); v[8 * q + 1] = bf16hi(w.x);
    v[8 * q + 2] = bf16lo(w.y); v[8 * q + 3] = bf16hi(w.y);
    v[8 * q + 4] = bf16lo(w.z); v[8 * q + 5] = bf16hi(w.z);
    v[8 * q + 6] = bf16lo(w.w); v[8 * q + 7] = bf16hi(w.w);
  }
}

template <>
__device__ __forceinline__ void load32<float>(const float* p, float* v) {
#pragma unroll
  for (int q = 0; q < 8; q++) {
    const float4 w = reinterpret_cast<const float4*>(p)[q];
    v[4 * q] = w.x; v[4 * q + 1] = w.y; v[4 * q + 2] = w.z; v[4 * q + 3] = w.w;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Row layout: one lane per 32-element block along a row (contiguous across the
// wave).  codes [rows][cols/2], scales [rows][cols/32].
// ---------------------------------------------------------------------------
template <typename T, int RND>
__global__ __launch_bounds__(256) void k_mx_cast_row(const T* __restrict__ x, int64_t rows,
                                                     int64_t cols, int64_t ld,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, uint32_t key) {
  const int64_t blocks = cols / 32;  // per row
  const int64_t it = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (it >= blocks) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    float v[32];
    load32<T>(x + r * ld + it * 32, v);
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 32; e++) am = fmaxf(am, fabsf(v[e]));
    uint32_t code;
    float mul;
    mx_scale(am, code, mul);
#pragma unroll
    for (int e = 0; e < 32; e++) v[e] *= mul;
    // whole lines per workgroup: non-temporal, like the NVFP4 row cast
    st_nt(codes + r * (cols / 2) + 16 * it, mx_encode32<RND>(v, key, (uint32_t)(r * cols + it * 32) >> 1));
    st_nt8(scales + r * blocks + it, (uint8_t)code);
  }
}

// ---------------------------------------------------------------------------
// Column layout: blocks of 32 consecutive rows of one column, written
// transposed.  A workgroup covers 512 rows x 64 columns; thread (g, co) loads
// 32 rows x 4 columns (8-byte bf16 row pieces, 16 threads per 128-byte line),
// encodes 4 column blocks and stages them in LDS so that each output row (one
// input column) is stored as contiguous 16-byte pieces.
// codes [cols][rows/2], scales [cols][rows/32].
// ---------------------------------------------------------------------------
constexpr int kMxTok = 512;
constexpr int kMxCols = 64;

template <typename T, int RND>
__global__ __launch_bounds__(256) void k_mx_cast_col(const T* __restrict__ x, int64_t rows,
                                                     int64_t cols, int64_t ld,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales, uint32_t key) {
  __shared__ __align__(16) uint8_t lcodes[kMxCols][kMxTok / 2];
  __shared__ __align__(16) uint8_t lscales[kMxCols][kMxTok / 32];
  const int64_t t0 = (int64_t)blockIdx.y * kMxTok;
  const int64_t c0 = (int64_t)blockIdx.x * kMxCols;
  const int co = threadIdx.x & 15;  // column quad
  const int g = threadIdx.x >> 4;   // 32-row block within the tile
  const int64_t tg = t0 + 32 * g;
  const int64_t cc = c0 + 4 * co;
  const bool valid = tg < rows && cc < cols;
  float u[4][32];
  if (valid) {
#pragma unroll
    for (int j = 0; j < 32; j++) {
      const T* p = x + (tg + j) * ld + cc;
      if constexpr (sizeof(T) == 2) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        u[0][j] = bf16lo(w.x); u[1][j] = bf16hi(w.x);
        u[2][j] = bf16lo(w.y); u[3][j] = bf16hi(w.y);
      } else {
        const float4 w = *reinterpret_cast<const float4*>(p);
        u[0][j] = w.x; u[1][j] = w.y; u[2][j] = w.z; u[3][j] = w.w;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; k++) {
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    uint32_t code = 0u;
    if (valid) {
      float am = 0.0f;
#pragma unroll
      for (int j = 0; j < 32; j++) am = fmaxf(am, fabsf(u[k][j]));
      float mul;
      mx_scale(am, code, mul);
#pragma unroll
      for (int j = 0; j < 32; j++) u[k][j] *= mul;
      w = mx_encode32<RND>(u[k], key, (uint32_t)((cc + k) * rows + tg) >> 1);
    }
    *reinterpret_cast<uint4*>(&lcodes[4 * co + k][16 * g]) = w;
    lscales[4 * co + k][g] = (uint8_t)code;
  }
  __syncthreads();
  // codes: 64 output rows of 256 bytes, 16 threads per row, 16 bytes each
  const int64_t row_bytes = rows / 2;
  for (int pass = 0; pass < 4; pass++) {
    const int lc = pass * 16 + (threadIdx.x >> 4);
    const int piece = threadIdx.x & 15;
    const int64_t c = c0 + lc;
    const int64_t off = t0 / 2 + 16 * piece;
    if (c < cols && off < row_bytes)
      st_nt(codes + c * row_bytes + off, *reinterpret_cast<const uint4*>(&lcodes[lc][16 * piece]));
  }
  // scales: 64 output rows of 16 bytes
  if (threadIdx.x < kMxCols) {
    const int lc = threadIdx.x;
    const int64_t c = c0 + lc;
    const int64_t srow = rows / 32;
    const int64_t off = t0 / 32;
    if (c < cols) {
      uint8_t* dst = scales + c * srow + off;
      const int n = (int)min((int64_t)16, srow - off);
      if (n == 16 && ((c * srow + off) & 15) == 0)
        st_nt(dst, *reinterpret_cast<const uint4*>(&lscales[lc][0]));
      else
        for (int b = 0; b < n; b++) st_nt8(dst + b, lscales[lc][b]);
    }
  }
}

static inline unsigned grid_cap_mx(int64_t want, int64_t cap) {
  if (want < 1) want = 1;
  return (unsigned)(want < cap ? want : cap);
}

hipError_t launch_mx_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int layout, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                              hipStream_t s) {
  const uint32_t key = sr_key(seed);
  if (layout == 0) {
    int64_t r = rows, c = cols, l = ld;
    if (ld == cols) {  // contiguous: one long row
      c = rows * cols;
      l = c;
      r = 1;
    }
    dim3 grid(grid_cap_mx((c / 32 + 255) / 256, 1 << 30), grid_cap_mx(r, 65535));
#define MXR(T, R) \
  k_mx_cast_row<T, R><<<grid, 256, 0, s>>>(static_cast<const T*>(x), r, c, l, codes, scales, key)
    if (dt == 0) {
      if (rnd == 0) MXR(uint16_t, 0); else MXR(uint16_t, 1);
    } else {
      if (rnd == 0) MXR(float, 0); else MXR(float, 1);
    }
#undef MXR
  } else {
    dim3 grid((unsigned)((cols + kMxCols - 1) / kMxCols), (unsigned)((rows + kMxTok - 1) / kMxTok));
#define MXC(T, R) \
  k_mx_cast_col<T, R><<<grid, 256, 0, s>>>(static_cast<const T*>(x), rows, cols, ld, codes, scales, key)
    if (dt == 0) {
      if (rnd == 0) MXC(uint16_t, 0); else MXC(uint16_t, 1);
    } else {
      if (rnd == 0) MXC(float, 0); else MXC(float, 1);
    }
#undef MXC
  }
  return hipGetLastError();
}

}  // namespace nvfp4
