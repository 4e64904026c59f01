// NVFP4 quantization kernels for gfx950: tensor amax, 1D row cast, 1D column
// cast (optionally after the 16x16 random Hadamard transform) and 2D 16x16
// tile cast with both orientations of the output.
//
// Method: "Pretraining Large Language Models with NVFP4" (gist.science
// summary), Resumo tecnico, 2. Metodologia Proposta -- "Formato NVFP4"
// (16-element blocks, E4M3 block scales, FP32 tensor scale) and techniques 2
// (random Hadamard transform on the Wgrad inputs), 3 (16x16 2D weight
// scaling) and 4 (stochastic rounding for gradients only).
//
// Every pass is bound by HBM bandwidth: loads are 16 bytes per lane and
// contiguous across a wave, block maxima are reduced in registers, and the
// column and tile casts stage their outputs through LDS so the transposed
// stores stay contiguous.  Each workgroup first tabulates S_enc / dec(e) for
// the 127 finite E4M3 codes in LDS, so a block scale costs one division by 6
// (a multiply and two FMAs) and one table read.
#include <algorithm>

#include "grid_sync.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"
#include "sync_ops.hpp"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Tensor amax
// ---------------------------------------------------------------------------

__global__ void k_zero_amax(float* amax, float* amax2) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    amax[0] = 0.0f;
    if (amax2 != nullptr) amax2[0] = 0.0f;
  }
}

// Most workgroups find a partial maximum below the running one: read it first
// (device-coherent) and skip the atomic, so thousands of workgroups do not
// serialize on one address.  The result is still the exact max.
__device__ __forceinline__ void atomic_max_if_larger(uint32_t r, float* amax) {
  unsigned int* a = reinterpret_cast<unsigned int*>(amax);
  if (r > __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) atomicMax(a, r);
}

// The workgroup's maxima of non-negative float bit patterns (m1 only if
// amax1 is not null) into the tensor amax outputs.  With an exchange slot the
// grid's maxima meet on its two-level lines (no workgroup waits) and the last
// workgroup to arrive writes both outputs, so the outputs need no clearing
// beforehand; without one (a stream under graph capture), one atomicMax each
// into outputs cleared by k_zero_amax.
__device__ __forceinline__ void block_atomic_max(uint32_t m0, float* amax0, uint32_t m1, float* amax1,
                                                 GridSyncSlot* slot) {
  __shared__ uint32_t red[2][8];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    m0 = max(m0, (uint32_t)__shfl_xor(m0, off));
    if (amax1 != nullptr) m1 = max(m1, (uint32_t)__shfl_xor(m1, off));
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[0][wave] = m0;
    red[1][wave] = m1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r0 = red[0][0], r1 = red[1][0];
    for (int w = 1; w < (int)(blockDim.x >> 6); w++) {
      r0 = max(r0, red[0][w]);
      r1 = max(r1, red[1][w]);
    }
    if (slot != nullptr) {
      const uint32_t G = gridDim.x * gridDim.y, id = blockIdx.y * gridDim.x + blockIdx.x;
      uint32_t t0 = 0u, t1 = 0u;
      if (grid_max_arrive<DeviceOps>(slot, G, id, r0, r1, &t0, &t1)) {
        DeviceOps::store_relaxed(reinterpret_cast<uint32_t*>(amax0), t0);
        if (amax1 != nullptr) DeviceOps::store_relaxed(reinterpret_cast<uint32_t*>(amax1), t1);
      }
    } else {
      atomic_max_if_larger(r0, amax0);
      if (amax1 != nullptr) atomic_max_if_larger(r1, amax1);
    }
  }
}

// amax over a rows x cols tensor with leading dimension ld (elements).  Each
// thread takes UNROLL 16-byte chunks per round, contiguous across the block.
template <typename T, int UNROLL>
__global__ __launch_bounds__(256) void k_amax(const T* __restrict__ x, int64_t rows, int64_t cols,
                                              int64_t ld, float* amax, GridSyncSlot* slot) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  const int64_t cpr = cols / EPC;       // chunks per row
  uint32_t m = 0u;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const uint4* row = reinterpret_cast<const uint4*>(x + r * ld);
    for (int64_t base = (int64_t)blockIdx.x * 256 * UNROLL; base < cpr;
         base += (int64_t)gridDim.x * 256 * UNROLL) {
      uint4 v[UNROLL];
#pragma unroll
      for (int j = 0; j < UNROLL; j++) {
        int64_t c = base + j * 256 + threadIdx.x;
        v[j] = c < cpr ? row[c] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < UNROLL; j++) {
        if constexpr (sizeof(T) == 2) {
          m = absmax_bf16x2(m, v[j].x);
          m = absmax_bf16x2(m, v[j].y);
          m = absmax_bf16x2(m, v[j].z);
          m = absmax_bf16x2(m, v[j].w);
        } else {
          uint32_t a = v[j].x & 0x7FFFFFFFu, b = v[j].y & 0x7FFFFFFFu;
          uint32_t c = v[j].z & 0x7FFFFFFFu, d = v[j].w & 0x7FFFFFFFu;
          a = a > b ? a : b;
          c = c > d ? c : d;
          a = a > c ? a : c;
          m = m > a ? m : a;
        }
      }
    }
  }
  if constexpr (sizeof(T) == 2) m <<= 16;
  block_atomic_max(m, amax, 0u, nullptr, slot);
}

// ---------------------------------------------------------------------------
// Element loads: 8 consecutive elements as FP32
// ---------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16lo(w.x); v[1] = bf16hi(w.x);
  v[2] = bf16lo(w.y); v[3] = bf16hi(w.y);
  v[4] = bf16lo(w.z); v[5] = bf16hi(w.z);
  v[6] = bf16lo(w.w); v[7] = bf16hi(w.w);
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Encode 16 scaled values (one block): RNE and SR through the hardware
// conversions, SR with pcg bits of output elements 2 pair0 .. 2 pair0 + 15
// (pair0 a multiple of 8).  Element 0 lands in the low nibble of x.
template <int RND>
__device__ __forceinline__ uint2 encode16(const float* v, uint32_t key, uint32_t pair0) {
  if constexpr (RND == 0) {
    return make_uint2(pack8_rne(v), pack8_rne(v + 8));
  } else {
    uint32_t h[8];
    pcg8(key, pair0, h);
    return make_uint2(sr_pack8(v, h), sr_pack8(v + 8, h + 4));
  }
}

// Encode 8 scaled values (half a block) into one dword, element 0 in the low
// nibble: RNE in hardware, SR with pcg bits of output elements 2 pair0 ..
// 2 pair0 + 7 (pair0 a multiple of 4).
template <int RND>
__device__ __forceinline__ uint32_t encode8(const float* v, uint32_t key, uint32_t pair0) {
  if constexpr (RND == 0) {
    return pack8_rne(v);
  } else {
    uint32_t h[4];
    pcg4(key, pair0, h);
    return sr_pack8(v, h);
  }
}

// Non-temporal output stores, where a workgroup writes whole contiguous lines
// (the row cast, the staged column stores, the 2D tile cast's transposed
// codes) or the rest of each line is written by a neighbour on the same XCD
// right after (the fused cast's row codes): the codes and scales are read
// next by another kernel (a GEMM), and dirty lines left in the caches would
// be written back while the next quantize call's amax pass streams its input.
// Partial lines from workgroups on different XCDs (the 2D tile cast's
// row-major codes, scale bytes) keep ordinary stores: non-temporal partial
// lines made those casts 8-41 % slower.

// ---------------------------------------------------------------------------
// 1D row cast: blocks of 16 along a row; each lane owns whole blocks (two
// 16-byte loads for bf16), UNROLL blocks per lane per round, contiguous
// across the workgroup.  codes [rows][cols/2], scales [rows][cols/16].
// ---------------------------------------------------------------------------
template <typename T, int RND, int UNROLL>
__global__ __launch_bounds__(256) void k_cast_row1d(const T* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld,
                                                    const float* __restrict__ amax,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales,
                                                    float* __restrict__ tensor_scale, uint32_t key) {
  __shared__ float rtab[128];
  const float s_enc = encode_scale(amax[0]);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) tensor_scale[0] = 1.0f / s_enc;
  fill_scale_table(rtab, s_enc);
  __syncthreads();
  const int64_t items = cols / 16;  // blocks per row
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const T* row = x + r * ld;
    uint2* crow = reinterpret_cast<uint2*>(codes + r * (cols / 2));
    uint8_t* srow = scales + r * (cols / 16);
    const uint32_t row_index = (uint32_t)(r * cols);
    for (int64_t base = (int64_t)blockIdx.x * 256 * UNROLL; base < items;
         base += (int64_t)gridDim.x * 256 * UNROLL) {
      float v[UNROLL][16];
#pragma unroll
      for (int j = 0; j < UNROLL; j++) {
        const int64_t it = base + j * 256 + threadIdx.x;
        if (it < items) {
          load8<T>(row + it * 16, v[j]);
          load8<T>(row + it * 16 + 8, v[j] + 8);
        } else {
#pragma unroll
          for (int e = 0; e < 16; e++) v[j][e] = 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < UNROLL; j++) {
        const int64_t it = base + j * 256 + threadIdx.x;
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < 16; e++) am = fmaxf(am, fabsf(v[j][e]));
        uint32_t e_b;
        float r_b;
        block_scale(am, s_enc, rtab, e_b, r_b);
        float sv[16];
#pragma unroll
        for (int e = 0; e < 16; e++) sv[e] = v[j][e] * r_b;
        if (it < items) {
          st_nt(&crow[it], encode16<RND>(sv, key, (row_index + (uint32_t)(it * 16)) >> 1));
          st_nt8(&srow[it], (uint8_t)e_b);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 1D column cast (COL_1D, and the Wgrad RHT path): blocks of 16 consecutive
// rows (tokens) in one column, written transposed.  A workgroup covers 256
// tokens x 128 columns: thread (g, co) loads 16 rows x 8 columns (16-byte
// row segments, 16 threads per 256-byte row piece), transforms and encodes
// its 8 column blocks, and stages codes and scales in LDS so each output row
// (one input column) gets one whole 128-byte line per workgroup.  The fused
// row + RHT kernel below writes its row copy straight from registers, 64
// bytes of codes per row per workgroup (a 512 x 64 tile gave 32-byte pieces).
// codes [cols][rows/2], scales [cols][rows/16].
// ---------------------------------------------------------------------------
constexpr int kColTok = 256;   // tokens per workgroup tile
constexpr int kColCols = 128;  // columns per workgroup tile
constexpr int kColOct = kColCols / 8;  // column octets (threads per 16-token group)
static_assert(kColOct * (kColTok / 16) == 256, "one thread per 16 tokens x 8 columns");
static_assert(kColTok >= 256, "col_store writes the scales as whole 16-byte pieces");

// A thread's 16 rows x 8 columns, kept as loaded (bf16: one 16-byte word per
// row, 64 VGPRs; fp32: two) and converted one column at a time, which keeps
// the register footprint (and so the occupancy) of the column kernels low.
template <typename T>
struct ColTile;

template <>
struct ColTile<uint16_t> {
  uint4 w[16];
  __device__ __forceinline__ void load(const uint16_t* p, int64_t ld) {
#pragma unroll
    for (int j = 0; j < 16; j++) w[j] = *reinterpret_cast<const uint4*>(p + j * ld);
  }
  // column k (0..7) of the 16 rows; with SIGN, row j's value negated where
  // bit j of sign_mask is set (the transform's sign flips)
  template <bool SIGN>
  __device__ __forceinline__ void column(int k, float* u, uint32_t sign_mask) const {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const uint32_t d = k < 2 ? w[j].x : k < 4 ? w[j].y : k < 6 ? w[j].z : w[j].w;
      const uint32_t sb = SIGN ? sign_bit(sign_mask, j) : 0u;
      u[j] = (k & 1) ? bf16hi_signed(d, sb) : bf16lo_signed(d, sb);
    }
  }
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int j = 0; j < 16; j++) asm volatile("" : "+v"(w[j].x), "+v"(w[j].y), "+v"(w[j].z), "+v"(w[j].w));
  }
  // the 8 values of row j
  __device__ __forceinline__ void row(int j, float* v) const {
    v[0] = bf16lo(w[j].x); v[1] = bf16hi(w[j].x); v[2] = bf16lo(w[j].y); v[3] = bf16hi(w[j].y);
    v[4] = bf16lo(w[j].z); v[5] = bf16hi(w[j].z); v[6] = bf16lo(w[j].w); v[7] = bf16hi(w[j].w);
  }
};

template <>
struct ColTile<float> {
  float4 w[16][2];
  __device__ __forceinline__ void load(const float* p, int64_t ld) {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      w[j][0] = *reinterpret_cast<const float4*>(p + j * ld);
      w[j][1] = *reinterpret_cast<const float4*>(p + j * ld + 4);
    }
  }
  template <bool SIGN>
  __device__ __forceinline__ void column(int k, float* u, uint32_t sign_mask) const {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const float4 q = w[j][k >> 2];
      const int e = k & 3;
      const float x = e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w;
      u[j] = SIGN ? f32_signed(x, sign_bit(sign_mask, j)) : x;
    }
  }
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int j = 0; j < 16; j++)
      for (int h = 0; h < 2; h++)
        asm volatile("" : "+v"(w[j][h].x), "+v"(w[j][h].y), "+v"(w[j][h].z), "+v"(w[j][h].w));
  }
  __device__ __forceinline__ void row(int j, float* v) const {
    v[0] = w[j][0].x; v[1] = w[j][0].y; v[2] = w[j][0].z; v[3] = w[j][0].w;
    v[4] = w[j][1].x; v[5] = w[j][1].y; v[6] = w[j][1].z; v[7] = w[j][1].w;
  }
};

// The column encoding of a tile (transform, block scale, encode) into the LDS
// staging arrays, and the contiguous stores of the staged codes and scales.
//
// FOLD (bf16 input, RHT only) leaves the 1/4 of the transform out of the 16
// values and puts it into the block's multiplier instead: the block maximum
// is 0.25 * max |u| (exact: rounding is monotone) and the scaled value is
// u * (0.25 * r_b).  That equals y * r_b with y = 0.25 u whenever both
// quarters are exact: 0.25 u always is for bf16 input (u is a multiple of
// 2^-133, so y is a multiple of 2^-135, never below the FP32 subnormal step),
// and 0.25 r_b is whenever r_b >= 2^-124 or r_b = 0, which S_enc >= 2^-100
// guarantees (r_b >= S_enc / 448).  The caller checks S_enc.
template <typename T, int RND, bool RHT, bool FOLD>
__device__ __forceinline__ void col_encode(const ColTile<T>& tile, int64_t rows, int64_t tg,
                                           int64_t cc, int g, int co, uint32_t sign_mask, float s_enc,
                                           const float* rtab, uint32_t key,
                                           uint8_t (*lcodes)[kColTok / 2],
                                           uint8_t (*lscales)[kColTok / 16]) {
  static_assert(!FOLD || (RHT && sizeof(T) == 2), "the 1/4 fold is exact for bf16 RHT input only");
#pragma unroll
  for (int k = 0; k < 8; k++) {
    float u[16];
    tile.template column<RHT>(k, u, sign_mask);
    if constexpr (FOLD)
      fwht16(u);
    else if constexpr (RHT)
      rht16_signed(u);
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; j++) am = fmaxf(am, fabsf(u[j]));
    if constexpr (FOLD) am = 0.25f * am;
    uint32_t e_b;
    float r_b;
    block_scale(am, s_enc, rtab, e_b, r_b);
    if constexpr (FOLD) r_b = 0.25f * r_b;
    float s[16];
#pragma unroll
    for (int j = 0; j < 16; j++) s[j] = u[j] * r_b;
    const uint2 w = encode16<RND>(s, key, (uint32_t)((cc + k) * rows + tg) >> 1);
    *reinterpret_cast<uint2*>(&lcodes[8 * co + k][8 * g]) = w;
    lscales[8 * co + k][g] = (uint8_t)e_b;
  }
}

// Whether the 1/4 of the transform may be folded into the block multipliers
// (see col_encode): bf16 input and S_enc >= 2^-100.
template <typename T>
__device__ __forceinline__ bool rht_fold_ok(float s_enc) {
  return sizeof(T) == 2 && s_enc >= 0x1p-100f;
}

template <typename T, int RND, bool RHT>
__device__ __forceinline__ void col_encode_any(const ColTile<T>& tile, int64_t rows, int64_t tg,
                                               int64_t cc, int g, int co, uint32_t sign_mask,
                                               float s_enc, const float* rtab, uint32_t key,
                                               uint8_t (*lcodes)[kColTok / 2],
                                               uint8_t (*lscales)[kColTok / 16]) {
  if constexpr (RHT && sizeof(T) == 2) {
    if (rht_fold_ok<T>(s_enc)) {  // uniform: one tensor scale
      col_encode<T, RND, true, true>(tile, rows, tg, cc, g, co, sign_mask, s_enc, rtab, key, lcodes,
                                     lscales);
      return;
    }
  }
  col_encode<T, RND, RHT, false>(tile, rows, tg, cc, g, co, sign_mask, s_enc, rtab, key, lcodes,
                                 lscales);
}

__device__ __forceinline__ void col_store(int64_t rows, int64_t cols, int64_t t0, int64_t c0,
                                          const uint8_t (*lcodes)[kColTok / 2],
                                          const uint8_t (*lscales)[kColTok / 16], uint8_t* codes,
                                          uint8_t* scales) {
  // codes: kColCols rows of kColTok / 2 bytes, 16 bytes per thread
  constexpr int kPieces = kColTok / 32;           // 16-byte pieces per row
  constexpr int kRowsPerPass = 256 / kPieces;
  const int64_t row_bytes = rows / 2;
  for (int pass = 0; pass < kColCols / kRowsPerPass; pass++) {
    int lc = pass * kRowsPerPass + (int)threadIdx.x / kPieces;  // local column
    int piece = (int)threadIdx.x % kPieces;
    int64_t c = c0 + lc;
    int64_t off = t0 / 2 + 16 * piece;  // byte offset within the output row
    if (c < cols && off < row_bytes) {
      uint8_t* dst = codes + c * row_bytes + off;
      const uint2* src = reinterpret_cast<const uint2*>(&lcodes[lc][16 * piece]);
      // row_bytes is a multiple of 8; 16-byte stores only where aligned
      if (off + 16 <= row_bytes && ((c * row_bytes + off) & 15) == 0) {
        st_nt(dst, *reinterpret_cast<const uint4*>(src));
      } else {
        st_nt(dst, src[0]);
        if (off + 16 <= row_bytes) st_nt(dst + 8, src[1]);
      }
    }
  }
  // scales: kColCols rows of kColTok / 16 bytes, 16 bytes per thread
  constexpr int kSPieces = kColTok / 256;
  if ((int)threadIdx.x < kColCols * kSPieces) {
    int lc = (int)threadIdx.x / kSPieces;
    int piece = (int)threadIdx.x % kSPieces;
    int64_t c = c0 + lc;
    const int64_t srow = rows / 16;
    int64_t off = t0 / 16 + 16 * piece;
    if (c < cols && off < srow) {
      uint8_t* dst = scales + c * srow + off;
      const uint8_t* src = &lscales[lc][16 * piece];
      if (off + 16 <= srow && ((c * srow + off) & 15) == 0) {
        st_nt(dst, *reinterpret_cast<const uint4*>(src));
      } else {
        for (int b = 0; b < 16 && off + b < srow; b++) st_nt8(dst + b, src[b]);
      }
    }
  }
}

template <typename T, int RND, bool RHT>
__global__ __launch_bounds__(256) void k_cast_col1d(const T* __restrict__ x, int64_t rows,
                                                    int64_t cols, int64_t ld, uint32_t sign_mask,
                                                    const float* __restrict__ amax,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales,
                                                    float* __restrict__ tensor_scale, uint32_t key) {
  __shared__ __align__(16) uint8_t lcodes[kColCols][kColTok / 2];
  __shared__ __align__(16) uint8_t lscales[kColCols][kColTok / 16];
  __shared__ float rtab[128];
  const float s_enc = encode_scale(amax[0]);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) tensor_scale[0] = 1.0f / s_enc;
  fill_scale_table(rtab, s_enc);
  __syncthreads();

  const int64_t t0 = (int64_t)blockIdx.y * kColTok;
  const int64_t c0 = (int64_t)blockIdx.x * kColCols;
  const int co = (int)threadIdx.x % kColOct;  // column octet
  const int g = (int)threadIdx.x / kColOct;   // 16-token group within the tile
  const int64_t tg = t0 + 16 * g;   // first token of the group
  const int64_t cc = c0 + 8 * co;   // first column of the octet
  // A thread whose 16 x 8 patch lies past the tensor loads the first patch
  // instead (in bounds: rows and cols are positive multiples of 16) and
  // encodes it into LDS slots that col_store never writes out.
  const bool valid = tg < rows && cc < cols;

  ColTile<T> tile;
  tile.load(valid ? x + tg * ld + cc : x, ld);
  col_encode_any<T, RND, RHT>(tile, rows, tg, cc, g, co, sign_mask, s_enc, rtab, key, lcodes, lscales);
  __syncthreads();
  col_store(rows, cols, t0, c0, lcodes, lscales, codes, scales);
}

// Row-1D copy and RHT column copy of the same tensor from ONE read (the two
// quantizations a training step needs from X or dY), with the column cast's
// tile mapping.  The row block of 16 columns spans the lane pair (co, co^1):
// each lane holds 8 of its values, one shuffle combines the two half maxima,
// and each lane encodes its 8 values (4 code bytes per row).
struct RowRhtArgs {
  int64_t rows, cols, ld;
  uint32_t sign_mask;
  uint8_t* row_codes;
  uint8_t* row_scales;
  uint32_t row_key;
  uint8_t* rht_codes;
  uint8_t* rht_scales;
  uint32_t rht_key;
};

// Where this thread's 16 x 8 patch of tile `id` (row-major over the
// 256-token x 128-column tiles) starts, and whether it lies in the tensor.
// The lane pair (co, co^1) agrees on validity (cols % 16 == 0); an invalid
// thread loads the first patch instead (in bounds) and stores nothing.
template <typename T>
__device__ __forceinline__ const T* row_rht_patch(const T* x, const RowRhtArgs& a, uint32_t id,
                                                  uint32_t tiles_x, bool& valid) {
  const int64_t tg = (int64_t)(id / tiles_x) * kColTok + 16 * ((int)threadIdx.x / kColOct);
  const int64_t cc = (int64_t)(id % tiles_x) * kColCols + 8 * ((int)threadIdx.x % kColOct);
  valid = tg < a.rows && cc < a.cols;
  return valid ? x + tg * a.ld + cc : x;
}

// Both encodings of one loaded tile.  Ends with every thread past its LDS
// reads, so the next tile may reuse the staging arrays.
template <typename T, int RR, int RH>
__device__ __forceinline__ void row_rht_tile(ColTile<T>& tile, bool valid, uint32_t id,
                                             uint32_t tiles_x, const RowRhtArgs& a, float s_row,
                                             float s_rht, const float* rtab_row,
                                             const float* rtab_rht,
                                             uint8_t (*lcodes)[kColTok / 2],
                                             uint8_t (*lscales)[kColTok / 16]) {
  const int64_t t0 = (int64_t)(id / tiles_x) * kColTok;
  const int64_t c0 = (int64_t)(id % tiles_x) * kColCols;
  const int co = (int)threadIdx.x % kColOct;
  const int g = (int)threadIdx.x / kColOct;
  const int64_t tg = t0 + 16 * g;
  const int64_t cc = c0 + 8 * co;

  // row copy: rows tg .. tg + 15, columns cc .. cc + 7 of this lane; the
  // output addresses and the hash index step by one row per iteration
  const int64_t rbytes = a.cols / 2, rscales = a.cols / 16;
  uint8_t* crow = a.row_codes + tg * rbytes + cc / 2;
  uint8_t* srow = a.row_scales + tg * rscales + cc / 16;
  uint32_t pair = (uint32_t)(tg * a.cols + cc) >> 1;  // elements < 2^32 (host check)
  const uint32_t pair_step = (uint32_t)a.cols >> 1;
#pragma unroll
  for (int j = 0; j < 16; j++) {
    float v[8];
    tile.row(j, v);
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; e++) am = fmaxf(am, fabsf(v[e]));
    am = fmaxf(am, __shfl_xor(am, 1));
    uint32_t e_b;
    float r_b;
    block_scale(am, s_row, rtab_row, e_b, r_b);
    float sv[8];
#pragma unroll
    for (int e = 0; e < 8; e++) sv[e] = v[e] * r_b;
    const uint32_t w = encode8<RR>(sv, a.row_key, pair);
    if (valid) {
      st_nt(crow, w);
      if ((co & 1) == 0) *srow = (uint8_t)e_b;
    }
    crow += rbytes;
    srow += rscales;
    pair += pair_step;
  }

  // RHT column copy.  The raw words pass through an empty asm first, so the
  // compiler converts them again one column at a time instead of keeping
  // the row copy's 128 converted values live (which costs ~50 VGPRs).
  tile.opaque();
  col_encode_any<T, RH, true>(tile, a.rows, tg, cc, g, co, a.sign_mask, s_rht, rtab_rht, a.rht_key,
                              lcodes, lscales);
  __syncthreads();
  col_store(a.rows, a.cols, t0, c0, lcodes, lscales, a.rht_codes, a.rht_scales);
  __syncthreads();
}

template <typename T>
__device__ __forceinline__ void row_rht_prologue(const float* row_amax, const float* rht_amax,
                                                 float* row_ts, float* rht_ts, float& s_row,
                                                 float& s_rht, float* rtab_row, float* rtab_rht) {
  s_row = encode_scale(row_amax[0]);
  s_rht = encode_scale(rht_amax[0]);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    row_ts[0] = 1.0f / s_row;
    rht_ts[0] = 1.0f / s_rht;
  }
  if (threadIdx.x < 128)
    rtab_row[threadIdx.x] = element_scale(threadIdx.x, s_row);
  else
    rtab_rht[threadIdx.x - 128] = element_scale(threadIdx.x - 128, s_rht);
  __syncthreads();
}

// Workgroup bid's place when each of the 8 XCDs (dealt workgroups
// round-robin by the hardware) takes a contiguous range of [0, G).
__device__ __forceinline__ uint32_t xcd_contiguous(uint32_t bid, uint32_t G) {
  const uint32_t xcd = bid & 7u, per = G >> 3, rem = G & 7u;
  return xcd < rem ? xcd * (per + 1) + (bid >> 3) : rem * (per + 1) + (xcd - rem) * per + (bid >> 3);
}

// One tile per workgroup.  XCD-aware tile order: the hardware deals
// workgroups round-robin over the 8 XCDs, so each XCD takes a contiguous
// range of tiles instead.  The two tiles that write the two halves of each
// row-copy line then run on the same XCD one after the other, and their
// halves meet in its L2.
template <typename T, int RR, int RH>
__global__ __launch_bounds__(256) void k_cast_row_rht(const T* __restrict__ x, RowRhtArgs a,
                                                      const float* __restrict__ row_amax,
                                                      float* __restrict__ row_ts,
                                                      const float* __restrict__ rht_amax,
                                                      float* __restrict__ rht_ts) {
  __shared__ __align__(16) uint8_t lcodes[kColCols][kColTok / 2];
  __shared__ __align__(16) uint8_t lscales[kColCols][kColTok / 16];
  __shared__ float rtab_row[128];
  __shared__ float rtab_rht[128];
  float s_row, s_rht;
  row_rht_prologue<T>(row_amax, rht_amax, row_ts, rht_ts, s_row, s_rht, rtab_row, rtab_rht);

  const uint32_t id = xcd_contiguous(blockIdx.y * gridDim.x + blockIdx.x, gridDim.x * gridDim.y);
  bool valid;
  ColTile<T> tile;
  tile.load(row_rht_patch(x, a, id, gridDim.x, valid), a.ld);
  row_rht_tile<T, RR, RH>(tile, valid, id, gridDim.x, a, s_row, s_rht, rtab_row, rtab_rht, lcodes,
                          lscales);
}

// Single-pass form of the fused call for a bf16 tensor that fits on chip
// (the tensor amax is needed before any block can be encoded, so the
// two-pass form reads the input twice).  The grid is at most the resident
// workgroup count (three per CU, up to 168 VGPRs per lane); the workgroup
// with place L (XCD-contiguous, as above) holds tiles [L * tiles / G,
// (L + 1) * tiles / G) of the 256 x 128 tiles, at most kRowRht1Tiles, in
// registers:
//   phase 1: both tiles' loads first, then the maxima of |x| and of the
//            unnormalized transform |u| over the workgroup's patches;
//   exchange: both maxima through grid_sync.hpp (bounded wait: a workgroup
//            that waits too long leaves its tiles to the publisher, the last
//            to arrive, which encodes them from memory after its own);
//   phase 2: the two-pass kernel's tile body on each held tile, so both
//            copies are identical to that path's.
// Round-to-nearest-even on both copies only: with stochastic rounding the
// encode is bound by its VALU work, which the two-pass form overlaps with
// the reads and this one cannot.
constexpr int kRowRht1Tiles = 2;

__global__ __launch_bounds__(256, 3) void k_row_rht_1pass(
    const uint16_t* __restrict__ x, RowRhtArgs a, uint32_t tiles, uint32_t tiles_x,
    float* __restrict__ row_ts, float* __restrict__ row_amax, float* __restrict__ rht_ts,
    float* __restrict__ rht_amax, GridSyncSlot* slot, uint32_t epoch, uint64_t spin_limit) {
  __shared__ __align__(16) uint8_t lcodes[kColCols][kColTok / 2];
  __shared__ __align__(16) uint8_t lscales[kColCols][kColTok / 16];
  __shared__ float rtab_row[128];
  __shared__ float rtab_rht[128];
  __shared__ uint32_t wave_max[2][4];
  __shared__ uint32_t sh_x, sh_u, sh_role, sh_n;
  const uint32_t G = gridDim.x;
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t L = xcd_contiguous(blockIdx.x, G);
  const uint32_t first = (uint32_t)((uint64_t)L * tiles / G);
  const uint32_t n = (uint32_t)((uint64_t)(L + 1) * tiles / G) - first;  // 1 or 2

  // phase 1: both loads first (a workgroup with one tile loads it twice, the
  // second copy in bounds and never used), then the two maxima.  Two named
  // tiles rather than an array: every access is then to a fixed register,
  // never to a stack copy.
  ColTile<uint16_t> t0, t1;
  bool v0, v1;
  t0.load(row_rht_patch(x, a, first, tiles_x, v0), a.ld);
  t1.load(row_rht_patch(x, a, first + n - 1u, tiles_x, v1), a.ld);
  v1 = v1 && n > 1u;
  float mx = 0.0f, mu = 0.0f;
  auto maxima = [&](const ColTile<uint16_t>& t) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      float u[16];
      t.template column<true>(k, u, a.sign_mask);  // sign flips do not change |x|
#pragma unroll
      for (int j = 0; j < 16; j++) mx = fmaxf(mx, fabsf(u[j]));
      fwht16(u);  // the 1/4 is applied once, to the maximum
#pragma unroll
      for (int j = 0; j < 16; j++) mu = fmaxf(mu, fabsf(u[j]));
    }
  };
  if (v0) maxima(t0);
  if (v1) maxima(t1);
  // keep the tiles in registers through the exchange (the loads are of
  // read-only memory, so the compiler would otherwise read them again)
  t0.opaque();
  t1.opaque();
  // non-negative floats: integer order is float order
  uint32_t bx = __float_as_uint(mx), bu = __float_as_uint(0.25f * mu);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    bx = max(bx, (uint32_t)__shfl_xor(bx, off));
    bu = max(bu, (uint32_t)__shfl_xor(bu, off));
  }
  if (lane == 0) {
    wave_max[0][tid >> 6] = bx;
    wave_max[1][tid >> 6] = bu;
  }
  __syncthreads();
  if (tid == 0) {
    const uint32_t wx = max(max(wave_max[0][0], wave_max[0][1]), max(wave_max[0][2], wave_max[0][3]));
    const uint32_t wu = max(max(wave_max[1][0], wave_max[1][1]), max(wave_max[1][2], wave_max[1][3]));
    uint32_t gx = 0u, gu = 0u, nrec = 0u;
    sh_role = grid_arrive_wait<DeviceOps>(slot, G, L, wx, epoch, spin_limit, &gx, &nrec, wu, &gu);
    sh_x = gx;
    sh_u = gu;
    sh_n = nrec;
  }
  __syncthreads();
  if (sh_role == kGridGaveUp) return;  // the publisher encodes this workgroup's tiles

  // phase 2: both encodings of every held tile
  const float amax_x = __uint_as_float(sh_x), amax_u = __uint_as_float(sh_u);
  const float s_row = encode_scale(amax_x), s_rht = encode_scale(amax_u);
  if (tid < 128)
    rtab_row[tid] = element_scale(tid, s_row);
  else
    rtab_rht[tid - 128] = element_scale(tid - 128, s_rht);
  __syncthreads();
  row_rht_tile<uint16_t, 0, 0>(t0, v0, first, tiles_x, a, s_row, s_rht, rtab_row, rtab_rht, lcodes,
                               lscales);
  if (n > 1u)
    row_rht_tile<uint16_t, 0, 0>(t1, v1, first + 1, tiles_x, a, s_row, s_rht, rtab_row, rtab_rht,
                                 lcodes, lscales);
  if (sh_role != kGridPublisher) return;

  // the publisher: the tensor outputs, and the tiles of the workgroups that
  // gave up, read again from memory
  if (tid == 0) {
    row_ts[0] = 1.0f / s_row;
    row_amax[0] = amax_x;
    rht_ts[0] = 1.0f / s_rht;
    rht_amax[0] = amax_u;
  }
  for (uint32_t i = 0; i < sh_n; i++) {
    __shared__ uint32_t sh_w;
    if (tid == 0) sh_w = grid_recovered<DeviceOps>(slot, i, uint64_t(1) << 22);
    __syncthreads();
    const uint32_t w = sh_w;
    __syncthreads();
    if (w >= G) continue;  // never stored (cannot happen: the entry follows its swap)
    const uint32_t f = (uint32_t)((uint64_t)w * tiles / G);
    const uint32_t e = (uint32_t)((uint64_t)(w + 1) * tiles / G);
    for (uint32_t id = f; id < e; id++) {
      bool ok;
      ColTile<uint16_t> one;
      one.load(row_rht_patch(x, a, id, tiles_x, ok), a.ld);
      row_rht_tile<uint16_t, 0, 0>(one, ok, id, tiles_x, a, s_row, s_rht, rtab_row, rtab_rht,
                                   lcodes, lscales);
    }
  }
}

// amax of the RHT output (and, if amax_plain is not null, of the input itself,
// from the same read).  A thread walks patches of 16 tokens x 4 columns (one
// 8-byte load per row for bf16), grid-stride, loading the next patch while it
// transforms the current one, so the reads stay in flight through the
// transform work.  Lane-consecutive patches are column-consecutive, so a wave
// reads 512 contiguous bytes per row.
template <typename T>
struct QuadTile;

template <>
struct QuadTile<uint16_t> {
  uint2 w[16];
  __device__ __forceinline__ void load(const uint16_t* p, int64_t ld) {
#pragma unroll
    for (int j = 0; j < 16; j++) w[j] = *reinterpret_cast<const uint2*>(p + j * ld);
  }
  // column k (0..3), row j negated where bit j of sign_mask is set
  __device__ __forceinline__ void column(int k, float* u, uint32_t sign_mask) const {
#pragma unroll
    for (int j = 0; j < 16; j++) {
      const uint32_t d = k < 2 ? w[j].x : w[j].y;
      const uint32_t sb = sign_bit(sign_mask, j);
      u[j] = (k & 1) ? bf16hi_signed(d, sb) : bf16lo_signed(d, sb);
    }
  }
};

template <>
struct QuadTile<float> {
  float4 w[16];
  __device__ __forceinline__ void load(const float* p, int64_t ld) {
#pragma unroll
    for (int j = 0; j < 16; j++) w[j] = *reinterpret_cast<const float4*>(p + j * ld);
  }
  __device__ __forceinline__ void column(int k, float* u, uint32_t sign_mask) const {
#pragma unroll
    for (int j = 0; j < 16; j++)
      u[j] = f32_signed(k == 0 ? w[j].x : k == 1 ? w[j].y : k == 2 ? w[j].z : w[j].w,
                        sign_bit(sign_mask, j));
  }
};

template <typename T>
__device__ __forceinline__ void rht_amax_patch(const QuadTile<T>& t, uint32_t sign_mask, bool plain,
                                               float& am, float& ap) {
#pragma unroll
  for (int k = 0; k < 4; k++) {
    float u[16];
    t.column(k, u, sign_mask);  // sign flips do not change |u|
    if (plain) {
#pragma unroll
      for (int j = 0; j < 16; j++) ap = fmaxf(ap, fabsf(u[j]));
    }
    fwht16(u);  // the 1/4 is applied once, to the maximum
#pragma unroll
    for (int j = 0; j < 16; j++) am = fmaxf(am, fabsf(u[j]));
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_rht_amax(const T* __restrict__ x, int64_t rows,
                                                  int64_t cols, int64_t ld, uint32_t sign_mask,
                                                  float* amax, float* amax_plain, GridSyncSlot* slot) {
  const uint32_t quads = (uint32_t)(cols / 4);            // column quads per 16-token band
  const uint32_t units = (uint32_t)(rows / 16) * quads;   // patches (< 2^26: elements < 2^32)
  const uint32_t stride = gridDim.x * 256u;
  const bool plain = amax_plain != nullptr;
  auto patch = [&](uint32_t p) {
    const uint32_t band = p / quads, q = p - band * quads;
    return x + (int64_t)band * 16 * ld + (int64_t)q * 4;
  };
  float am = 0.0f, ap = 0.0f;
  uint32_t p = blockIdx.x * 256u + threadIdx.x;
  QuadTile<T> ta, tb;
  if (p < units) ta.load(patch(p), ld);
  while (p < units) {
    const uint32_t pb = p + stride;
    if (pb < units) tb.load(patch(pb), ld);
    rht_amax_patch(ta, sign_mask, plain, am, ap);
    if (pb >= units) break;
    const uint32_t pa = pb + stride;
    if (pa < units) ta.load(patch(pa), ld);
    rht_amax_patch(tb, sign_mask, plain, am, ap);
    p = pa;
  }
  // max |RN(u / 4)| = RN(max |u| / 4): rounding is monotone
  am = 0.25f * am;
  block_atomic_max(__float_as_uint(am), amax, __float_as_uint(ap), amax_plain, slot);
}

// 16 consecutive elements as loaded (bf16: two 16-byte words; fp32: four),
// converted to FP32 on use.
template <typename T>
struct Raw16;

template <>
struct Raw16<uint16_t> {
  uint4 w[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    w[0] = reinterpret_cast<const uint4*>(p)[0];
    w[1] = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ void get(float* v) const {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      v[8 * h + 0] = bf16lo(w[h].x); v[8 * h + 1] = bf16hi(w[h].x);
      v[8 * h + 2] = bf16lo(w[h].y); v[8 * h + 3] = bf16hi(w[h].y);
      v[8 * h + 4] = bf16lo(w[h].z); v[8 * h + 5] = bf16hi(w[h].z);
      v[8 * h + 6] = bf16lo(w[h].w); v[8 * h + 7] = bf16hi(w[h].w);
    }
  }
};

template <>
struct Raw16<float> {
  float4 w[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int q = 0; q < 4; q++) w[q] = reinterpret_cast<const float4*>(p)[q];
  }
  __device__ __forceinline__ void get(float* v) const {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      v[4 * q + 0] = w[q].x; v[4 * q + 1] = w[q].y; v[4 * q + 2] = w[q].z; v[4 * q + 3] = w[q].w;
    }
  }
};

// ---------------------------------------------------------------------------
// 2D tile cast: one scale per 16x16 tile.  A workgroup covers 256 rows x 64
// columns in four passes; in pass j wave w takes tile row 4j + w, lane l holds
// row l%16 of tile column l/16 (16 elements).  The tile amax is reduced over the 16 lanes of
// a tile.  Row-major codes go straight out (8 bytes per lane, 4 lanes per
// 32-byte row piece).  The transposed codes are the same codes (one scale per
// tile) read down the columns: the 16 lanes of a tile transpose their 16 x 16
// nibble matrix in registers (below), and the packed columns are staged in LDS
// so that each row of codes_t gets a whole 128-byte line per workgroup.
// codes [rows][cols/2], scales [rows/16][cols/16],
// codes_t [cols][rows/2], scales_t [cols/16][rows/16].
// ---------------------------------------------------------------------------

// Lane-xor exchange within each group of 32 lanes (ds_swizzle bit mode).
template <int XOR>
__device__ __forceinline__ uint32_t swz_xor(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (XOR << 10) | 0x1F);
}

// Transpose of a 16 x 16 matrix of nibbles held by 16 consecutive lanes: on
// entry lane r holds row r (nibble c of the 64-bit w1:w0 = column c), on exit
// column r.  Four butterfly stages exchange ever smaller blocks between lanes
// r and r ^ d (d = 8, 4, 2, 1): the upper-right block of each pair of rows
// swaps with the lower-left one.
__device__ __forceinline__ void transpose16x16_nibbles(uint32_t& w0, uint32_t& w1, int r) {
  // d = 8: 8 x 8 blocks (whole words)
  {
    const bool hi = r & 8;
    const uint32_t got = swz_xor<8>(hi ? w0 : w1);
    if (hi) w0 = got; else w1 = got;
  }
  // d = 4: 4 x 4 blocks (16-bit halves of both words)
  {
    const bool hi = r & 4;
    const uint32_t send = hi ? ((w0 & 0xFFFFu) | (w1 << 16)) : ((w0 >> 16) | (w1 & 0xFFFF0000u));
    const uint32_t got = swz_xor<4>(send);
    if (hi) {
      w0 = (w0 & 0xFFFF0000u) | (got & 0xFFFFu);
      w1 = (w1 & 0xFFFF0000u) | (got >> 16);
    } else {
      w0 = (w0 & 0xFFFFu) | (got << 16);
      w1 = (w1 & 0xFFFFu) | (got & 0xFFFF0000u);
    }
  }
  // d = 2: 2 x 2 blocks (bytes 1, 3 of the low lane <-> bytes 0, 2 of the high)
  {
    const bool hi = r & 2;
    // v_perm(a, b, sel): selector byte values 0..3 take b's bytes, 4..7 a's
    const uint32_t send = hi ? __builtin_amdgcn_perm(w1, w0, 0x06040200u)   // w0.b0, w0.b2, w1.b0, w1.b2
                             : __builtin_amdgcn_perm(w1, w0, 0x07050301u);  // w0.b1, w0.b3, w1.b1, w1.b3
    const uint32_t got = swz_xor<2>(send);  // the partner's four bytes, same order
    if (hi) {
      w0 = __builtin_amdgcn_perm(w0, got, 0x07010500u);  // got.b0, w0.b1, got.b1, w0.b3
      w1 = __builtin_amdgcn_perm(w1, got, 0x07030502u);  // got.b2, w1.b1, got.b3, w1.b3
    } else {
      w0 = __builtin_amdgcn_perm(got, w0, 0x05020400u);  // w0.b0, got.b0, w0.b2, got.b1
      w1 = __builtin_amdgcn_perm(got, w1, 0x07020600u);  // w1.b0, got.b2, w1.b2, got.b3
    }
  }
  // d = 1: single nibbles (high nibbles of the even lane <-> low nibbles of the odd)
  {
    const bool hi = r & 1;
    const uint32_t lo4 = 0x0F0F0F0Fu;
    const uint32_t send = hi ? ((w0 & lo4) | ((w1 & lo4) << 4)) : (((w0 >> 4) & lo4) | (w1 & ~lo4));
    const uint32_t got = swz_xor<1>(send);
    if (hi) {
      w0 = (w0 & ~lo4) | (got & lo4);
      w1 = (w1 & ~lo4) | ((got >> 4) & lo4);
    } else {
      w0 = (w0 & lo4) | ((got & lo4) << 4);
      w1 = (w1 & lo4) | (got & ~lo4);
    }
  }
}

template <typename T, int RND>
__global__ __launch_bounds__(256) void k_cast_tile2d(const T* __restrict__ x, int64_t rows,
                                                     int64_t cols, int64_t ld,
                                                     const float* __restrict__ amax,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     uint8_t* __restrict__ codes_t,
                                                     uint8_t* __restrict__ scales_t,
                                                     float* __restrict__ tensor_scale, uint32_t key) {
  __shared__ __align__(16) uint8_t lt[64][128];  // [local column][packed codes of the 256 rows]
  __shared__ __align__(16) uint8_t lsc[16][4];   // [tile row][tile column] scale codes
  __shared__ float rtab[128];
  const float s_enc = encode_scale(amax[0]);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) tensor_scale[0] = 1.0f / s_enc;
  fill_scale_table(rtab, s_enc);
  __syncthreads();

  // consecutive workgroups take consecutive row regions of one column strip
  const int64_t r0 = (int64_t)blockIdx.x * 256;
  const int64_t c0 = (int64_t)blockIdx.y * 64;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int tc = lane >> 4;  // tile column in the region
  const int rr = lane & 15;  // row within the tile
  const int64_t c = c0 + 16 * tc;

  // The four tile rows 4j + wave of the region (16 rows each): all their
  // loads are issued first (a tile outside the tensor reads the tensor's
  // first 16 elements instead and stores nothing), then each is encoded.
  Raw16<T> raw[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int64_t r = r0 + 16 * (4 * j + wave) + rr;
    const bool tile_valid = (r0 + 16 * (4 * j + wave)) < rows && c < cols;
    raw[j].load(tile_valid ? x + r * ld + c : x);
  }
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int tr = 4 * j + wave;
    const int64_t r = r0 + 16 * tr + rr;
    const bool tile_valid = (r0 + 16 * tr) < rows && c < cols;  // whole tile in or out
    float v[16];
    raw[j].get(v);
    float am = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; e++) am = fmaxf(am, fabsf(v[e]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) am = fmaxf(am, __shfl_xor(am, off));
    uint32_t e_b;
    float r_b;
    block_scale(am, s_enc, rtab, e_b, r_b);
    float sv[16];
#pragma unroll
    for (int e = 0; e < 16; e++) sv[e] = v[e] * r_b;
    const uint2 w = encode16<RND>(sv, key, (uint32_t)(r * cols + c) >> 1);
    uint32_t w0 = w.x, w1 = w.y;
    if (tile_valid) *reinterpret_cast<uint2*>(codes + r * (cols / 2) + c / 2) = make_uint2(w0, w1);
    if (rr == 0) lsc[tr][tc] = (uint8_t)e_b;  // stored below, where the tile is in the tensor
    if (codes_t != nullptr) {
      // every lane of the wave takes part in the exchange (an invalid tile's
      // codes land in staging slots that are never stored)
      transpose16x16_nibbles(w0, w1, rr);
      // lane (tc, rr) now holds column c + rr of the tile's 16 rows
      *reinterpret_cast<uint2*>(&lt[16 * tc + rr][8 * tr]) = make_uint2(w0, w1);
    }
  }
  __syncthreads();
  // Scale codes from LDS in whole pieces (single bytes from every tile would
  // each leave the L2 as a partial write): a row of `scales` gets the
  // region's 4 codes as one dword, a row of `scales_t` its 16 as 16 bytes.
  {
    const int64_t nr = rows / 16, nc = cols / 16, br0 = r0 / 16, bc0 = c0 / 16;
    const int t = (int)threadIdx.x;
    if (t < 16 && br0 + t < nr) {
      uint8_t* dst = scales + (br0 + t) * nc + bc0;
      const int n = (int)min((int64_t)4, nc - bc0);
      if (n == 4 && (((br0 + t) * nc + bc0) & 3) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = *reinterpret_cast<const uint32_t*>(lsc[t]);
      } else {
        for (int k = 0; k < n; k++) dst[k] = lsc[t][k];
      }
    } else if (scales_t != nullptr && t >= 64 && t < 68 && bc0 + (t - 64) < nc) {
      const int q = t - 64;
      uint8_t* dst = scales_t + (bc0 + q) * nr + br0;
      const int n = (int)min((int64_t)16, nr - br0);
      uint32_t wv[4];
#pragma unroll
      for (int k = 0; k < 4; k++)
        wv[k] = (uint32_t)lsc[4 * k][q] | ((uint32_t)lsc[4 * k + 1][q] << 8) |
                ((uint32_t)lsc[4 * k + 2][q] << 16) | ((uint32_t)lsc[4 * k + 3][q] << 24);
      if (n == 16 && (((bc0 + q) * nr + br0) & 15) == 0) {
        *reinterpret_cast<uint4*>(dst) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
      } else {
        for (int k = 0; k < n; k++) dst[k] = (uint8_t)(wv[k >> 2] >> (8 * (k & 3)));
      }
    }
  }
  if (codes_t == nullptr) return;
  // codes_t: 64 rows (local columns) of up to 128 bytes; 4 threads per row,
  // each storing 16-byte pieces q and q + 4, so each store instruction covers
  // 64 contiguous bytes of a row (non-temporal stores are not merged in L2:
  // pieces with gaps between them would each leave as a partial write)
  const int lc = threadIdx.x >> 2;
  const int q = threadIdx.x & 3;
  const int64_t ct = c0 + lc;
  if (ct >= cols) return;
  const int64_t row_bytes = rows / 2;
#pragma unroll
  for (int k = 0; k < 2; k++) {
    const int piece = 4 * k + q;
    const int64_t off = r0 / 2 + 16 * piece;  // byte offset in the output row
    if (off >= row_bytes) break;
    uint8_t* dst = codes_t + ct * row_bytes + off;
    const uint8_t* src = &lt[lc][16 * piece];
    if (off + 16 <= row_bytes && ((ct * row_bytes + off) & 15) == 0) {
      st_nt(dst, *reinterpret_cast<const uint4*>(src));
    } else {  // row_bytes is a multiple of 8
      st_nt(dst, reinterpret_cast<const uint2*>(src)[0]);
      if (off + 16 <= row_bytes) st_nt(dst + 8, reinterpret_cast<const uint2*>(src)[1]);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static inline unsigned grid_cap(int64_t want, int64_t cap) {
  if (want < 1) want = 1;
  return (unsigned)(want < cap ? want : cap);
}

// Compute units of the current device (256, the MI355X count, if the query
// fails).
static int cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}

// Without an exchange slot for the stream (graph capture) the outputs are
// cleared first and every workgroup maxes into them atomically.
template <typename T>
static hipError_t launch_amax(const void* x, int64_t rows, int64_t cols, int64_t ld, float* amax,
                              hipStream_t s) {
  GridSyncSlot* slot = stream_sync_slot(s);
  if (slot == nullptr) k_zero_amax<<<1, 64, 0, s>>>(amax, nullptr);
  constexpr int EPC = 16 / sizeof(T);
  constexpr int UNROLL = 8;
  if (ld == cols) {  // contiguous: one long row
    cols = rows * cols;
    ld = cols;
    rows = 1;
  }
  int64_t cpr = cols / EPC;
  // one long row: four workgroups per compute unit walking the tensor in
  // rounds (measured: 1.3x the rate of twice as many on an 84 MB tensor);
  // strided rows: at most 2048 workgroups per row, rounds balanced
  const int64_t units = (cpr + 256 * UNROLL - 1) / (256 * UNROLL);
  dim3 grid;
  if (rows == 1) {
    grid = dim3(grid_cap(units, 4 * (int64_t)cu_count()), 1);
  } else {
    const int64_t rounds = (units + 2047) / 2048;
    grid = dim3(grid_cap((units + rounds - 1) / rounds, 2048), grid_cap(rows, 65535));
  }
  k_amax<T, UNROLL><<<grid, 256, 0, s>>>(static_cast<const T*>(x), rows, cols, ld, amax, slot);
  return hipGetLastError();
}

// The cast pass of nvfp4_quantize (amax already final).
static hipError_t launch_cast(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int layout, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                              uint8_t* codes_t, uint8_t* scales_t, float* tensor_scale,
                              float* amax, hipStream_t s) {
  const uint32_t key = sr_key(seed);
  if (layout == 0) {
    constexpr int UNROLL = 2;
    int64_t r = rows, c = cols, l = ld;
    if (ld == cols) {
      c = rows * cols;
      l = c;
      r = 1;
    }
    int64_t items = c / 16;
    dim3 grid(grid_cap((items + 256 * UNROLL - 1) / (256 * UNROLL), 1 << 20), grid_cap(r, 65535));
#define ROW_LAUNCH(T, R)                                                                        \
  k_cast_row1d<T, R, UNROLL><<<grid, 256, 0, s>>>(static_cast<const T*>(x), r, c, l, amax, codes, \
                                                  scales, tensor_scale, key)
    if (dt == 0) {
      if (rnd == 0) ROW_LAUNCH(uint16_t, 0); else ROW_LAUNCH(uint16_t, 1);
    } else {
      if (rnd == 0) ROW_LAUNCH(float, 0); else ROW_LAUNCH(float, 1);
    }
#undef ROW_LAUNCH
  } else if (layout == 1) {
    dim3 grid((unsigned)((cols + kColCols - 1) / kColCols), (unsigned)((rows + kColTok - 1) / kColTok));
#define COL_LAUNCH(T, R)                                                                          \
  k_cast_col1d<T, R, false><<<grid, 256, 0, s>>>(static_cast<const T*>(x), rows, cols, ld, 0u, amax, \
                                                 codes, scales, tensor_scale, key)
    if (dt == 0) {
      if (rnd == 0) COL_LAUNCH(uint16_t, 0); else COL_LAUNCH(uint16_t, 1);
    } else {
      if (rnd == 0) COL_LAUNCH(float, 0); else COL_LAUNCH(float, 1);
    }
#undef COL_LAUNCH
  } else {
    dim3 grid((unsigned)((rows + 255) / 256), (unsigned)((cols + 63) / 64));
#define TILE_LAUNCH(T, R)                                                                  \
  k_cast_tile2d<T, R><<<grid, 256, 0, s>>>(static_cast<const T*>(x), rows, cols, ld, amax, \
                                           codes, scales, codes_t, scales_t, tensor_scale, key)
    if (dt == 0) {
      if (rnd == 0) TILE_LAUNCH(uint16_t, 0); else TILE_LAUNCH(uint16_t, 1);
    } else {
      if (rnd == 0) TILE_LAUNCH(float, 0); else TILE_LAUNCH(float, 1);
    }
#undef TILE_LAUNCH
  }
  return hipGetLastError();
}

// Workgroups of k_rht_amax that fit on the current device at once.
template <typename T>
static int rht_amax_occupancy() {
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_rht_amax<T>, 256, 0) != hipSuccess) n = 0;
    return n;
  }();
  return occ;
}

static int64_t rht_amax_resident(int dt) {
  const int occ = dt == 0 ? rht_amax_occupancy<uint16_t>() : rht_amax_occupancy<float>();
  return (int64_t)std::max(occ, 1) * cu_count();
}

// RHT amax pass (plus the plain amax into amax_plain when it is not null).
static hipError_t launch_rht_amax(const void* x, int dt, int64_t tokens, int64_t cols, int64_t ld,
                                  uint32_t sign_mask, float* amax, float* amax_plain, hipStream_t s) {
  GridSyncSlot* slot = stream_sync_slot(s);
  if (slot == nullptr) k_zero_amax<<<1, 64, 0, s>>>(amax, amax_plain);
  // patches of 16 tokens x 4 columns, at most one grid of resident
  // workgroups walking them (A/B on one box: 8192x5120 RHT call 42.6 -> 41.5
  // us, 8192x20480 SR 171.3 -> 165.5 us, against balanced rounds of up to
  // 2048 workgroups, which leave a partial last round of workgroups)
  const int64_t units = (tokens / 16) * (cols / 4);
  const int64_t wgs = (units + 255) / 256;
  const unsigned grid = grid_cap(std::min<int64_t>(wgs, rht_amax_resident(dt)), 2048);
  if (dt == 0)
    k_rht_amax<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), tokens, cols, ld,
                                              sign_mask, amax, amax_plain, slot);
  else
    k_rht_amax<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), tokens, cols, ld, sign_mask,
                                           amax, amax_plain, slot);
  return hipGetLastError();
}

// The cast pass of nvfp4_rht_quantize (amax already final).
static hipError_t launch_rht_cast(const void* x, int dt, int64_t tokens, int64_t cols, int64_t ld,
                                  uint32_t sign_mask, int rnd, uint64_t seed, uint8_t* codes,
                                  uint8_t* scales, float* tensor_scale, float* amax, hipStream_t s) {
  dim3 grid((unsigned)((cols + kColCols - 1) / kColCols), (unsigned)((tokens + kColTok - 1) / kColTok));
  const uint32_t key = sr_key(seed);
#define RHT_LAUNCH(T, R)                                                                         \
  k_cast_col1d<T, R, true><<<grid, 256, 0, s>>>(static_cast<const T*>(x), tokens, cols, ld,       \
                                                sign_mask, amax, codes, scales, tensor_scale, key)
  if (dt == 0) {
    if (rnd == 0) RHT_LAUNCH(uint16_t, 0); else RHT_LAUNCH(uint16_t, 1);
  } else {
    if (rnd == 0) RHT_LAUNCH(float, 0); else RHT_LAUNCH(float, 1);
  }
#undef RHT_LAUNCH
  return hipGetLastError();
}

hipError_t launch_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                           int layout, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                           uint8_t* codes_t, uint8_t* scales_t, float* tensor_scale, float* amax,
                           hipStream_t s) {
  if (layout == 0) {
    bool done = false;
    hipError_t e = try_quantize_row_1pass(x, dt, rows, cols, ld, rnd, seed, codes, scales,
                                          tensor_scale, amax, s, &done);
    if (e != hipSuccess || done) return e;
  }
  hipError_t e = dt == 0 ? launch_amax<uint16_t>(x, rows, cols, ld, amax, s)
                         : launch_amax<float>(x, rows, cols, ld, amax, s);
  if (e != hipSuccess) return e;
  return launch_cast(x, dt, rows, cols, ld, layout, rnd, seed, codes, scales, codes_t, scales_t,
                     tensor_scale, amax, s);
}

hipError_t launch_rht_quantize(const void* x, int dt, int64_t tokens, int64_t cols, int64_t ld,
                               uint32_t sign_mask, int rnd, uint64_t seed, uint8_t* codes,
                               uint8_t* scales, float* tensor_scale, float* amax, hipStream_t s) {
  sign_mask &= 0xFFFFu;
  hipError_t e = launch_rht_amax(x, dt, tokens, cols, ld, sign_mask, amax, nullptr, s);
  if (e != hipSuccess) return e;
  return launch_rht_cast(x, dt, tokens, cols, ld, sign_mask, rnd, seed, codes, scales, tensor_scale,
                         amax, s);
}

// Workgroups of k_row_rht_1pass that fit on one compute unit.
static int row_rht_1pass_occupancy() {
  static const int occ = [] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_row_rht_1pass, 256, 0) != hipSuccess) n = 0;
    return n;
  }();
  return occ;
}

// The single-pass fused call where it applies (bf16 input, RNE on both
// copies, tiles that fit in the resident grid's registers, an exchange slot
// free); *done = false and nothing enqueued otherwise.
static hipError_t try_row_rht_1pass(const void* x, int dt, uint32_t tiles_x, uint32_t tiles_y,
                                    int row_rnd, int rht_rnd, const RowRhtArgs& a, float* row_ts,
                                    float* row_amax, float* rht_ts, float* rht_amax,
                                    hipStream_t s, bool* done) {
  *done = false;
  if (dt != 0 || row_rnd != 0 || rht_rnd != 0) return hipSuccess;
  const int occ = row_rht_1pass_occupancy();
  if (occ < 1) return hipSuccess;
  const int64_t tiles = (int64_t)tiles_x * tiles_y;
  const int64_t resident = std::min<int64_t>((int64_t)occ * cu_count(), kSyncMaxGrid);
  if (tiles > resident * kRowRht1Tiles) return hipSuccess;  // does not fit on chip
  SinglePassTicket tk;
  if (!single_pass_ticket(s, &tk)) return hipSuccess;
  // every resident workgroup (more loads in flight), each with one or two tiles
  const unsigned grid = (unsigned)std::min<int64_t>(resident, tiles);
  k_row_rht_1pass<<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), a, (uint32_t)tiles, tiles_x,
                                       row_ts, row_amax, rht_ts, rht_amax, tk.slot, tk.epoch, tk.spin);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  *done = true;
  single_pass_launched(tk);
  return hipSuccess;
}

// Both quantizations of one tensor: in one pass where the tensor fits on
// chip, else one read for the two amaxes, then the row cast and the RHT
// column cast.
hipError_t launch_quantize_row_rht(const void* x, int dt, int64_t tokens, int64_t cols, int64_t ld,
                                   int row_rnd, uint64_t row_seed, uint8_t* row_codes,
                                   uint8_t* row_scales, float* row_ts, float* row_amax,
                                   uint32_t sign_mask, int rht_rnd, uint64_t rht_seed,
                                   uint8_t* rht_codes, uint8_t* rht_scales, float* rht_ts,
                                   float* rht_amax, hipStream_t s) {
  sign_mask &= 0xFFFFu;
  const uint32_t tiles_x = (uint32_t)((cols + kColCols - 1) / kColCols);
  const uint32_t tiles_y = (uint32_t)((tokens + kColTok - 1) / kColTok);
  const RowRhtArgs a{tokens, cols, ld, sign_mask, row_codes, row_scales, sr_key(row_seed),
                     rht_codes, rht_scales, sr_key(rht_seed)};
  bool done = false;
  hipError_t e = try_row_rht_1pass(x, dt, tiles_x, tiles_y, row_rnd, rht_rnd, a, row_ts, row_amax,
                                   rht_ts, rht_amax, s, &done);
  if (e != hipSuccess || done) return e;
  e = launch_rht_amax(x, dt, tokens, cols, ld, sign_mask, rht_amax, row_amax, s);
  if (e != hipSuccess) return e;
  // both casts from one read of x
#define ROW_RHT_LAUNCH(T, RR, RH)                                                                 \
  k_cast_row_rht<T, RR, RH><<<dim3(tiles_x, tiles_y), 256, 0, s>>>(static_cast<const T*>(x), a,   \
                                                                row_amax, row_ts, rht_amax, rht_ts)
#define ROW_RHT_RND(T)                                             \
  if (row_rnd == 0) {                                              \
    if (rht_rnd == 0) { ROW_RHT_LAUNCH(T, 0, 0); } else { ROW_RHT_LAUNCH(T, 0, 1); } \
  } else {                                                         \
    if (rht_rnd == 0) { ROW_RHT_LAUNCH(T, 1, 0); } else { ROW_RHT_LAUNCH(T, 1, 1); } \
  }
  if (dt == 0) {
    ROW_RHT_RND(uint16_t)
  } else {
    ROW_RHT_RND(float)
  }
#undef ROW_RHT_RND
#undef ROW_RHT_LAUNCH
  return hipGetLastError();
}

}  // namespace nvfp4
