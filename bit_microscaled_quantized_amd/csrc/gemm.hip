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
// values is exact in FP32.  Each wave dequantizes its operand fragments in
// registers (hardware FP4->F16 conversion, then a packed FP16 multiply by the
// block scale), contracts them on the FP16 matrix cores
// (v_mfma_f32_32x32x16_f16, FP32 accumulation) and applies the two FP32
// tensor scales once in the epilogue.  The only rounding is the FP32
// accumulation and the final alpha multiply.  One MFMA step covers 16
// K-elements, i.e. exactly one scale block per operand row.
//
// Data movement: the operands stay 4.5 bits per element all the way into LDS.
// A stage covers 256 K-elements: 128 code bytes (one full 128-byte line) and
// 16 scale bytes per row, for the workgroup's 256 A rows and 256 B rows
// (72 KB); two stages are double-buffered (144 KB of the 160 KB LDS).  Stages
// are fetched with direct-to-LDS loads (global_load_lds, 16 bytes per lane for
// codes, 4 for scales) issued one stage ahead, so no registers hold prefetched
// data and each code load instruction covers eight full cache lines.  Chunk c
// (16 bytes) of row r lands in slot 8r + (c ^ (r & 7)), which makes the
// fragment reads (32 consecutive rows, same chunk) bank-conflict free.
//
// Tiling: 512 threads = 8 waves (two per SIMD, so one wave's conversions
// overlap the other's MFMAs) in a 2 x 4 grid; workgroup tile 256 x 256, wave
// tile 128 x 64 = 4 x 2 MFMA tiles of 32 x 32 (128 FP32 accumulators per
// lane).  Inside a stage K is permuted so that one 16-byte chunk read feeds
// four MFMA steps: lane half h reads chunks 4h .. 4h + 3 of its row; in quad g
// (chunk 4h + g) step s uses the chunk's dword s, i.e. stage elements
// 32(4h + g) + 8s .. + 7, identically for A and B, which leaves the
// contraction unchanged.  Rows past M/N and chunks past K are fetched from
// clamped in-row addresses; past K the scales are zeroed (exact 0
// contribution), past M/N the outputs are never stored.  Workgroups are
// remapped so that each XCD's share of the grid is a contiguous, grouped range
// of output tiles (shared L2).
#include <mutex>

#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BKS = 256;                           // K elements per stage
constexpr int CODE_BYTES = BM * (BKS / 2);         // 32 KB per operand
constexpr int SCALE_BYTES = BM * (BKS / 16);       // 4 KB per operand
constexpr int OFF_B = CODE_BYTES;                  // B codes
constexpr int OFF_SA = 2 * CODE_BYTES;             // A scales
constexpr int OFF_SB = 2 * CODE_BYTES + SCALE_BYTES;
constexpr int STAGE_BYTES = 2 * CODE_BYTES + 2 * SCALE_BYTES;  // 72 KB
constexpr int LDS_BYTES = 2 * STAGE_BYTES;                     // 144 KB

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// Each lane's `size` bytes at g land at l + lane * size (l wave-uniform).
__device__ __forceinline__ void load_lds16(const uint8_t* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((gvoid*)g, (lvoid*)l, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const uint8_t* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((gvoid*)g, (lvoid*)l, 4, 0, 0);
}

// 8 FP4 codes -> 8 FP16 values times the block scale s (exact).
__device__ __forceinline__ half8_t dequant8(uint32_t w, half2_t s) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ uint32_t dw(const uint4& q, int i) {
  return i == 0 ? q.x : i == 1 ? q.y : i == 2 ? q.z : q.w;
}

}  // namespace

__global__ __launch_bounds__(512, 1) void k_gemm_nvfp4(
    int M, int N, int K, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, int b_rowdiv, const float* __restrict__ b_ts,
    float* __restrict__ c, int64_t ldc, int accumulate) {
  extern __shared__ __align__(16) uint8_t lds[];

  // XCD-aware tile order: the hardware deals workgroups round-robin over the
  // 8 XCDs, so gather each XCD's share into a contiguous range of tiles, then
  // walk the tiles in groups of GROUP tile rows.
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int64_t kb = K / 2;   // code bytes per row (a multiple of 32)
  const int64_t ks = K / 16;  // scale bytes per row (a multiple of 4)
  const int KT = (K + BKS - 1) / BKS;

  // ---- stage fetch.  Code instruction j of a wave: rows 8(4 wave + j) + l/8,
  // lane l takes chunk (l%8) ^ (row & 7) of its row.  Scale instruction i:
  // rows 32 wave + 16 i + l/4, lane l takes dword l%4 of the row's 16 bytes.
  const int crow = lane >> 3;
  const int cchunk = (lane & 7) ^ crow;
  const int sdw = lane & 3;
  auto issue_stage = [&](int kt, uint8_t* st) {
    // in-row byte offsets, clamped to the row's last chunk / dword
    const int64_t coff = min((int64_t)kt * (BKS / 2) + 16 * cchunk, kb - 16);
    const int64_t soff = min((int64_t)kt * (BKS / 16) + 4 * sdw, ks - 4);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int r = 8 * (4 * wave + j) + crow;
      load_lds16(a_codes + (int64_t)min(m0 + r, M - 1) * kb + coff, st + (4 * wave + j) * 1024);
      load_lds16(b_codes + (int64_t)min(n0 + r, N - 1) * kb + coff, st + OFF_B + (4 * wave + j) * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int r = 32 * wave + 16 * i + (lane >> 2);
      load_lds4(a_scales + (int64_t)min(m0 + r, M - 1) * ks + soff, st + OFF_SA + (2 * wave + i) * 256);
      load_lds4(b_scales + (int64_t)(min(n0 + r, N - 1) / b_rowdiv) * ks + soff,
                st + OFF_SB + (2 * wave + i) * 256);
    }
  };
  // In a stage that ends past K, zero the scale bytes of blocks >= K/16: their
  // codes and scales came from clamped addresses and must contribute exactly 0.
  auto fix_partial = [&](int kt, uint8_t* st) {
    const int valid = (int)min((int64_t)BKS / 16, ks - (int64_t)kt * (BKS / 16));
    if (valid >= BKS / 16) return;
    uint8_t* row = st + (tid < 256 ? OFF_SA + tid * 16 : OFF_SB + (tid - 256) * 16);
    for (int i = valid; i < 16; i++) row[i] = 0;
  };

  // ---- fragment reads.  Lane (h, lr) of A tile i reads row wm*128 + 32i + lr
  // (B tile j: row wn*64 + 32j + lr), chunk 4h + g in quad g: slot
  // 8*row + ((4h + g) ^ (lr & 7)); its two scale bytes (blocks 2(4h + g) and
  // 2(4h + g) + 1) sit at row*16 + 2(4h + g).
  const int rowa = wm * 128 + lr;
  const int rowb = wn * 64 + lr;
  auto read_quad = [&](const uint8_t* st, int g, uint4* ca, uint4* cb, uint32_t* sa, uint32_t* sb) {
    const int sw = ((4 * h + g) ^ (lr & 7)) << 4;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      ca[i] = *reinterpret_cast<const uint4*>(st + (rowa + 32 * i) * 128 + sw);
      sa[i] = *reinterpret_cast<const uint16_t*>(st + OFF_SA + (rowa + 32 * i) * 16 + 2 * (4 * h + g));
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
      cb[j] = *reinterpret_cast<const uint4*>(st + OFF_B + (rowb + 32 * j) * 128 + sw);
      sb[j] = *reinterpret_cast<const uint16_t*>(st + OFF_SB + (rowb + 32 * j) * 16 + 2 * (4 * h + g));
    }
  };

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  // quad data double-buffered by quad parity
  uint4 qa[2][4], qb[2][2];
  uint32_t qsa[2][4], qsb[2][2];

  // 4 MFMA steps on the quad in buffer p: per step, convert the 6 fragments
  // (48 VALU) and issue 8 MFMAs; the other wave on the SIMD overlaps them
  auto quad = [&](int p) {
    half2_t sca[4][2], scb[2][2];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      half2_t v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qsa[p][i], 1.0f, false);
      sca[i][0] = half2_t{v[0], v[0]};
      sca[i][1] = half2_t{v[1], v[1]};
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
      half2_t v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(qsb[p][j], 1.0f, false);
      scb[j][0] = half2_t{v[0], v[0]};
      scb[j][1] = half2_t{v[1], v[1]};
    }
#pragma unroll
    for (int s = 0; s < 4; s++) {
      half8_t fa[4], fb[2];
#pragma unroll
      for (int i = 0; i < 4; i++) fa[i] = dequant8(dw(qa[p][i], s), sca[i][s >> 1]);
#pragma unroll
      for (int j = 0; j < 2; j++) fb[j] = dequant8(dw(qb[p][j], s), scb[j][s >> 1]);
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  };

  // prologue: stage 0 in buffer 0, its quad 0 read
  issue_stage(0, lds);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  fix_partial(0, lds);
  __syncthreads();
  read_quad(lds, 0, qa[0], qb[0], qsa[0], qsb[0]);

  for (int kt = 0; kt < KT; kt++) {
    uint8_t* cur = lds + (kt & 1) * STAGE_BYTES;
    uint8_t* nxt = lds + ((kt + 1) & 1) * STAGE_BYTES;
    const bool more = kt + 1 < KT;
    if (more) issue_stage(kt + 1, nxt);
    // quads 0..2: read the following quad of this stage while computing
#pragma unroll
    for (int g = 0; g < 3; g++) {
      const int p = g & 1;
      read_quad(cur, g + 1, qa[p ^ 1], qb[p ^ 1], qsa[p ^ 1], qsb[p ^ 1]);
      quad(p);
    }
    // quad 3 (buffer 1): the next stage becomes visible, its quad 0 is read
    // into buffer 0 while this stage's last quad is computed, and a final
    // barrier releases this stage's LDS buffer for the next prefetch.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (more) {
      const int valid = (int)min((int64_t)BKS / 16, ks - (int64_t)(kt + 1) * (BKS / 16));
      if (valid < BKS / 16) {
        fix_partial(kt + 1, nxt);
        __syncthreads();
      }
      read_quad(nxt, 0, qa[0], qb[0], qsa[0], qsb[0]);
    }
    quad(1);
    __syncthreads();
  }

  const float alpha = a_ts[0] * b_ts[0];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const int n = n0 + wn * 64 + j * 32 + lr;
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
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_nvfp4),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  k_gemm_nvfp4<<<(unsigned)tiles, 512, LDS_BYTES, s>>>((int)M, (int)N, (int)K, a_codes, a_scales,
                                                       a_ts, b_codes, b_scales, b_rowdiv, b_ts, c,
                                                       ldc, accumulate);
  return hipGetLastError();
}

}  // namespace nvfp4
