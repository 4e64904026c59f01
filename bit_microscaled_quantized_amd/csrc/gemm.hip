// NVFP4 block-scaled GEMM for gfx950:
//   C = beta * C + (a_ts * b_ts) * sum_k (qA * eA) (qB * eB)
// with A [M][K/2] and B [N][K/2] packed E2M1 codes (K contiguous, "NT"),
// E4M3 scales per 16 K-elements, and one FP32 tensor scale per operand.
//
// Method: "Pretraining Large Language Models with NVFP4" (gist.science
// summary), Resumo tecnico, 2. Metodologia Proposta ("Formato NVFP4", the
// two-level scales) and 3. Contribuicoes ("Suporte de Hardware": GEMMs run on
// the NVFP4 operands directly).
//
// Exactness: an E2M1 value (<= 2 significant bits) times an E4M3 scale
// (<= 4 significant bits, 2^-9 .. 448) has at most 6 significant bits and
// lies in [2^-10, 2688], so it is exact in FP16, and the product of two such
// values is exact in FP32.  The kernel therefore folds each block scale into
// its operand while converting FP4 -> FP16 in registers (hardware FP4->F16
// conversion, then a packed FP16 multiply by the scale), contracts on the FP16
// matrix cores (v_mfma_f32_32x32x16_f16, FP32 accumulation) and applies the
// two FP32 tensor scales once in the epilogue.  The only rounding is the FP32
// accumulation and the final alpha multiply.
//
// Tiling: 256 threads = 4 waves in a 2x2 grid; workgroup tile 256 x 256, wave
// tile 128 x 128 = 4 x 4 MFMA tiles of 32 x 32 (256 FP32 accumulators per
// lane); K advances 64 per stage.  Per stage the raw FP4 codes (32 bytes per
// row) and the scales (converted once to FP16) are staged in LDS, double
// buffered with one barrier per stage.  K is permuted inside a stage so every
// lane reads its 32 codes as one 16-byte LDS load: lane half h = lane / 32,
// k-step s, element e hold stage element 32h + 8s + e, identically for A and
// B, which leaves the contraction unchanged.  Workgroups are remapped so that
// neighbouring output tiles run on the same XCD (shared L2).
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;          // K elements per stage
constexpr int ROWB = BK / 2;    // code bytes per row per stage (32)
constexpr int NSB = BK / 16;    // scale blocks per row per stage (4)

struct __align__(16) Stage {
  uint8_t a[BM * ROWB];        // [BM/32][2][32][16 B]
  uint8_t b[BN * ROWB];
  _Float16 sa[BM * NSB];       // [BM][4]
  _Float16 sb[BN * NSB];
};

__device__ __forceinline__ int code_slot(int row, int h) {
  return ((row >> 5) << 10) + (h << 9) + ((row & 31) << 4);
}

__device__ __forceinline__ uint64_t scales_to_f16x4(uint32_t w) {
  uint64_t r = 0;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    _Float16 h = (_Float16)e4m3_decode((w >> (8 * i)) & 0xFFu);
    r |= (uint64_t)__builtin_bit_cast(uint16_t, h) << (16 * i);
  }
  return r;
}

// 8 FP4 codes (one dword, element 0 in the low nibble) -> 8 FP16 values times
// the block scale s (exact).
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  p0 = p0 * s;
  p1 = p1 * s;
  p2 = p2 * s;
  p3 = p3 * s;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

struct Prefetch {
  uint4 a[2], b[2];
  uint32_t sa, sb;
};

}  // namespace

__global__ __launch_bounds__(256, 1) void k_gemm_nvfp4(
    int M, int N, int K, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, int b_rowdiv, const float* __restrict__ b_ts,
    float* __restrict__ c, int64_t ldc, int accumulate) {
  __shared__ Stage st[2];

  // XCD-aware tile order: the hardware deals workgroups round-robin over the
  // 8 XCDs, so gather each XCD's share into a contiguous range of tiles.
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, per = G >> 3, rem = G & 7;
  const int id = (xcd < rem) ? xcd * (per + 1) + (bid >> 3) : rem * (per + 1) + (xcd - rem) * per + (bid >> 3);
  const int num_m = (M + BM - 1) / BM;
  const int num_n = (N + BN - 1) / BN;
  constexpr int GROUP = 8;
  const int width = GROUP * num_n;
  const int first_m = (id / width) * GROUP;
  const int gsz = min(num_m - first_m, GROUP);
  const int pm = first_m + (id % width) % gsz;
  const int pn = (id % width) / gsz;
  const int m0 = pm * BM, n0 = pn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t kb = K / 2;    // code bytes per row
  const int64_t ks = K / 16;   // scale bytes per row

  // global -> register prefetch of one stage
  auto load_stage = [&](int kt, Prefetch& p) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      int q = tid + 256 * i;
      int row = q >> 1, h = q & 1;
      int64_t off = (int64_t)kt * ROWB + 16 * h;
      p.a[i] = (m0 + row < M) ? *reinterpret_cast<const uint4*>(a_codes + (int64_t)(m0 + row) * kb + off)
                              : make_uint4(0, 0, 0, 0);
      p.b[i] = (n0 + row < N) ? *reinterpret_cast<const uint4*>(b_codes + (int64_t)(n0 + row) * kb + off)
                              : make_uint4(0, 0, 0, 0);
    }
    p.sa = (m0 + tid < M) ? *reinterpret_cast<const uint32_t*>(a_scales + (int64_t)(m0 + tid) * ks + kt * NSB) : 0u;
    p.sb = (n0 + tid < N)
               ? *reinterpret_cast<const uint32_t*>(b_scales + (int64_t)((n0 + tid) / b_rowdiv) * ks + kt * NSB)
               : 0u;
  };
  auto store_stage = [&](Stage& s, const Prefetch& p) {
#pragma unroll
    for (int i = 0; i < 2; i++) {
      int q = tid + 256 * i;
      int row = q >> 1, h = q & 1;
      *reinterpret_cast<uint4*>(s.a + code_slot(row, h)) = p.a[i];
      *reinterpret_cast<uint4*>(s.b + code_slot(row, h)) = p.b[i];
    }
    *reinterpret_cast<uint64_t*>(s.sa + tid * NSB) = scales_to_f16x4(p.sa);
    *reinterpret_cast<uint64_t*>(s.sb + tid * NSB) = scales_to_f16x4(p.sb);
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  const int KT = K / BK;
  Prefetch pf;
  load_stage(0, pf);
  store_stage(st[0], pf);
  __syncthreads();

  const int h = lane >> 5;
  const int lr = lane & 31;
  for (int kt = 0; kt < KT; kt++) {
    if (kt + 1 < KT) load_stage(kt + 1, pf);
    const Stage& s = st[kt & 1];
    uint4 ca[4], cb[4];
    half2_t sa[4][2], sb[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      int ra = wm * 128 + i * 32 + lr;
      int rb = wn * 128 + i * 32 + lr;
      ca[i] = *reinterpret_cast<const uint4*>(s.a + code_slot(ra, h));
      cb[i] = *reinterpret_cast<const uint4*>(s.b + code_slot(rb, h));
      half2_t pa = *reinterpret_cast<const half2_t*>(s.sa + ra * NSB + 2 * h);
      half2_t pb = *reinterpret_cast<const half2_t*>(s.sb + rb * NSB + 2 * h);
      sa[i][0] = half2_t{pa[0], pa[0]};
      sa[i][1] = half2_t{pa[1], pa[1]};
      sb[i][0] = half2_t{pb[0], pb[0]};
      sb[i][1] = half2_t{pb[1], pb[1]};
    }
#pragma unroll
    for (int st_ = 0; st_ < 4; st_++) {
      half8_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        uint32_t wa = st_ == 0 ? ca[i].x : st_ == 1 ? ca[i].y : st_ == 2 ? ca[i].z : ca[i].w;
        uint32_t wb = st_ == 0 ? cb[i].x : st_ == 1 ? cb[i].y : st_ == 2 ? cb[i].z : cb[i].w;
        fa[i] = dequant8(wa, sa[i][st_ >> 1]);
        fb[i] = dequant8(wb, sb[i][st_ >> 1]);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_stage(st[(kt + 1) & 1], pf);
    __syncthreads();
  }

  const float alpha = a_ts[0] * b_ts[0];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int n = n0 + wn * 128 + j * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (m < M && n < N) {
          float* p = c + (int64_t)m * ldc + n;
          float v = alpha * acc[i][j][r];
          if (accumulate) v += *p;
          *p = v;
        }
      }
    }
}

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_ts, const uint8_t* b_codes,
                       const uint8_t* b_scales, int b_rowdiv, const float* b_ts, float* c,
                       int64_t ldc, int accumulate, hipStream_t s) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  k_gemm_nvfp4<<<(unsigned)tiles, 256, 0, s>>>((int)M, (int)N, (int)K, a_codes, a_scales, a_ts,
                                                b_codes, b_scales, b_rowdiv, b_ts, c, ldc, accumulate);
  return hipGetLastError();
}

}  // namespace nvfp4
