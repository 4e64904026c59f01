// MXFP4 GEMM (the comparison format): C = beta * C + sum_k (qA * 2^eA)(qB * 2^eB)
// with A [M][K/2], B [N][K/2] E2M1 codes and E8M0 scales [rows][K/32].
//
// gfx950 has a matrix instruction for exactly this format:
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands takes each lane's 32
// codes (one row, one 32-element block: lane l holds row l % 32 and K half
// l / 32 of the instruction's 64) and that block's E8M0 scale, and accumulates
// the exact products in FP32 -- no conversion instructions at all.  With no
// conversions to overlap, one wave per SIMD suffices: 256 threads = 4 waves
// (2 x 2), wave tile 128 x 128 = 4 x 4 MFMA tiles (256 accumulators in AGPRs,
// 16 MFMAs per step).  Workgroup tile (256 x 256), staging (raw codes through
// direct-to-LDS loads, swizzled 16-byte chunks) and tail split are those of
// the NVFP4 kernel (gemm_tiling.hpp); a stage holds 256 K-elements (4 MFMA
// steps) and 8 scale bytes per row.  Per stage each lane reads its rows' 8
// scale bytes once and regroups them (one byte permute) so that byte s is the
// scale of its block in step s, selected by the instruction's op_sel.
//
// Format: "Pretraining Large Language Models with NVFP4" (gist.science
// summary), Resumo tecnico, parts 1 and 2 (MXFP4, the format NVFP4 is
// compared with: 32-element blocks, power-of-two UE8M0 scales, no tensor
// scale).
#include <mutex>

#include "gemm_tiling.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {
namespace {
constexpr int MX_SCALE_BYTES = BM * (BKS / 32);                     // 2 KB per operand
constexpr int MX_OFF_SA = 2 * CODE_BYTES;
constexpr int MX_OFF_SB = 2 * CODE_BYTES + MX_SCALE_BYTES;
constexpr int MX_STAGE_BYTES = 2 * CODE_BYTES + 2 * MX_SCALE_BYTES;  // 68 KB
constexpr int MX_LDS_BYTES = 2 * MX_STAGE_BYTES;                     // 136 KB
typedef int int4v_t __attribute__((ext_vector_type(4)));
typedef int int8v_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ int8v_t fp4_operand(const int4v_t& v) {
  return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);  // FP4 reads 4 registers
}
}  // namespace

__global__ __launch_bounds__(256, 1) void k_gemm_mxfp4(
    int M, int N, int K, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ b_codes, const uint8_t* __restrict__ b_scales,
    float* __restrict__ c, int64_t ldc, int accumulate, int full_tiles, int split,
    float* __restrict__ partial) {
  extern __shared__ __align__(16) uint8_t lds[];

  const int KT = (K + BKS - 1) / BKS;
  const int bid = blockIdx.x;
  int id, kt0 = 0, kt1 = KT;
  float* part = nullptr;
  if (bid < full_tiles) {
    const int G = full_tiles;
    const int xcd = bid & 7, per = G >> 3, rem = G & 7;
    id = (xcd < rem) ? xcd * (per + 1) + (bid >> 3) : rem * (per + 1) + (xcd - rem) * per + (bid >> 3);
  } else {
    const int u = bid - full_tiles;
    const int q = u % split;
    id = full_tiles + u / split;
    kt0 = (int)((int64_t)KT * q / split);
    kt1 = (int)((int64_t)KT * (q + 1) / split);
    part = partial + (int64_t)u * (BM * BN);
  }
  const int num_m = (M + BM - 1) / BM;
  const int num_n = (N + BN - 1) / BN;
  int pm, pn;
  tile_of(id, num_m, num_n, pm, pn);
  const int m0 = pm * BM, n0 = pn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int64_t kb = K / 2;   // code bytes per row (a multiple of 64)
  const int64_t ks = K / 32;  // scale bytes per row (a multiple of 4)

  // ---- stage fetch.  Code instruction j (0..7) of wave w: rows
  // r = 8(8w + j) + l/8, lane l fills slot l%8, i.e. takes chunk
  // (l%8) ^ ((r >> 1) & 7) = (l%8) ^ (4 (j & 1) + (l/8) / 2).  Scale
  // instruction i (0..1): rows 64w + 32i + l/2, dword l%2 of the row's 8 bytes.
  const int crow = lane >> 3;
  const int cchunk_e = (lane & 7) ^ (crow >> 1);
  const int cchunk_o = (lane & 7) ^ (4 + (crow >> 1));
  const int sdw = lane & 1;
  auto issue_stage = [&](int kt, uint8_t* st) __attribute__((always_inline)) {
    const int64_t coff_e = min((int64_t)kt * (BKS / 2) + 16 * cchunk_e, kb - 16);
    const int64_t coff_o = min((int64_t)kt * (BKS / 2) + 16 * cchunk_o, kb - 16);
    const int64_t soff = min((int64_t)kt * (BKS / 32) + 4 * sdw, ks - 4);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const int r = 8 * (8 * wave + j) + crow;
      const int64_t coff = (j & 1) ? coff_o : coff_e;
      load_lds16(a_codes + (int64_t)min(m0 + r, M - 1) * kb + coff, st + (8 * wave + j) * 1024);
      load_lds16(b_codes + (int64_t)min(n0 + r, N - 1) * kb + coff, st + OFF_B + (8 * wave + j) * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int r = 64 * wave + 32 * i + (lane >> 1);
      load_lds4(a_scales + (int64_t)min(m0 + r, M - 1) * ks + soff, st + MX_OFF_SA + (2 * wave + i) * 256);
      load_lds4(b_scales + (int64_t)min(n0 + r, N - 1) * ks + soff, st + MX_OFF_SB + (2 * wave + i) * 256);
    }
  };
  // In a stage that ends past K (K is a multiple of 128, so only its second
  // half can be past the end), zero the codes of the last 128 K-elements
  // (chunks 4..7) of every row: exact zero contributions whatever the scale.
  auto fix_partial = [&](int kt, uint8_t* st) __attribute__((always_inline)) {
    if ((int64_t)(kt + 1) * BKS <= K) return;
    const int f = (tid >> 1) & 7;  // row tid of A and of B
#pragma unroll
    for (int cidx = 4; cidx < 8; cidx++) {
      *reinterpret_cast<uint4*>(st + tid * 128 + ((cidx ^ f) << 4)) = make_uint4(0u, 0u, 0u, 0u);
      *reinterpret_cast<uint4*>(st + OFF_B + tid * 128 + ((cidx ^ f) << 4)) = make_uint4(0u, 0u, 0u, 0u);
    }
  };

  // ---- fragment reads: step s of a stage uses chunk 2s + h of the lane's rows
  const int rowa = wm * 128 + lr;
  const int rowb = wn * 128 + lr;
  const int fsw = (lr >> 1) & 7;
  // (native vector loads: one load per fragment whose address derives from
  // the stage buffer alone, so it keeps that buffer's alias scope and is not
  // made to wait for the prefetch into the other buffer)
  auto read_step = [&](const uint8_t* __restrict__ st, int s, int4v_t* ca, int4v_t* cb) __attribute__((always_inline)) {
    const int sw = ((2 * s + h) ^ fsw) << 4;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      ca[i] = *reinterpret_cast<const int4v_t*>(st + (rowa + 32 * i) * 128 + sw);
      cb[i] = *reinterpret_cast<const int4v_t*>(st + OFF_B + (rowb + 32 * i) * 128 + sw);
    }
  };
  // this lane's scale dword for each of its rows: byte s = block 2s + h
  const uint32_t psel = h ? 0x07050301u : 0x06040200u;
  auto read_scales = [&](const uint8_t* __restrict__ st, uint32_t* sa, uint32_t* sb) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const uint2 wa = *reinterpret_cast<const uint2*>(st + MX_OFF_SA + (rowa + 32 * i) * 8);
      const uint2 wb = *reinterpret_cast<const uint2*>(st + MX_OFF_SB + (rowb + 32 * i) * 8);
      sa[i] = __builtin_amdgcn_perm(wa.y, wa.x, psel);
      sb[i] = __builtin_amdgcn_perm(wb.y, wb.x, psel);
    }
  };

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  int4v_t qa[2][4], qb[2][4];
  uint32_t sa[2][4], sb[2][4];  // scale dwords of the current / next stage

// 16 MFMAs of step S on fragment buffer P; the scheduling barrier keeps the
// reads of step S + 1 overlapping these MFMAs
#define MX_MFMAS(P, S)                                                                           \
  _Pragma("unroll") for (int i = 0; i < 4; i++) _Pragma("unroll") for (int j = 0; j < 4; j++)   \
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(                               \
          fp4_operand(qa[P][i]), fp4_operand(qb[P][j]), acc[i][j], 4, 4, S, sa[0][i], S,       \
          sb[0][j]);                                                                            \
  __builtin_amdgcn_sched_barrier(0);

  issue_stage(kt0, lds);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  fix_partial(kt0, lds);
  __syncthreads();
  read_scales(lds, sa[0], sb[0]);
  read_step(lds, 0, qa[0], qb[0]);

  // One stage; cur and nxt are the two disjoint stage buffers (restrict: the
  // fragment reads of cur do not wait for the prefetch into nxt).  After the
  // barrier that publishes nxt, no wave reads cur again, so the next
  // iteration may refill it without a second barrier.
  auto stage = [&](int kt, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
    const bool more = kt + 1 < kt1;
    // issued on the last stage too (clamped, in-row addresses; the data goes
    // unused): without the branch around it the compiler interleaves the 20
    // loads with this stage's first MFMAs and waits less before them
    issue_stage(kt + 1, nxt);
    read_step(cur, 1, qa[1], qb[1]);
    MX_MFMAS(0, 0)
    read_step(cur, 2, qa[0], qb[0]);
    MX_MFMAS(1, 1)
    read_step(cur, 3, qa[1], qb[1]);
    MX_MFMAS(0, 2)
    // keep these MFMAs above the barrier (the compiler would otherwise sink
    // them past it, leaving the matrix core idle through the barrier wait)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) asm volatile("" : "+a"(acc[i][j]));
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (more) {
      if ((int64_t)(kt + 2) * BKS > K) {
        fix_partial(kt + 1, nxt);
        __syncthreads();
      }
      read_scales(nxt, sa[1], sb[1]);
      read_step(nxt, 0, qa[0], qb[0]);
    }
    MX_MFMAS(1, 3)
#pragma unroll
    for (int i = 0; i < 4; i++) {
      sa[0][i] = sa[1][i];
      sb[0][i] = sb[1][i];
    }
  };
  for (int kt = kt0; kt < kt1; kt++) {
    uint8_t* cur = lds + ((kt - kt0) & 1) * MX_STAGE_BYTES;
    uint8_t* nxt = lds + ((kt - kt0 + 1) & 1) * MX_STAGE_BYTES;
    stage(kt, cur, nxt);
  }
#undef MX_MFMAS

  // Epilogue, one 32 x 32 tile (16 stores per lane) at a time: the scheduling
  // barriers keep the compiler from computing all 256 store addresses up
  // front, which would not fit in the VGPRs left beside the accumulators.
  if (part != nullptr) {
    float* pb = part + (wm * 128 + 4 * h) * BN + wn * 128 + lr;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
#pragma unroll
        for (int r = 0; r < 16; r++) pb[(i * 32 + 8 * (r >> 2) + (r & 3)) * BN + j * 32] = acc[i][j][r];
        __builtin_amdgcn_sched_barrier(0);
      }
    return;
  }
  const int mb = m0 + wm * 128 + 4 * h;
  const int nb = n0 + wn * 128 + lr;
  float* cb = c + (int64_t)mb * ldc + nb;
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const bool n_ok = nb + j * 32 < N;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int dm = i * 32 + 8 * (r >> 2) + (r & 3);
        if (n_ok && mb + dm < M) {
          float* p = cb + (int64_t)dm * ldc + j * 32;
          float v = acc[i][j][r];
          if (accumulate) v += *p;
          __builtin_nontemporal_store(v, p);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
}


hipError_t launch_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                          const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                          float* c, int64_t ldc, int accumulate, void* workspace,
                          int64_t workspace_bytes, hipStream_t s) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_mxfp4),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, MX_LDS_BYTES);
  });
  if (attr_err != hipSuccess) return attr_err;
  SplitPlan p = plan_split(M, N, K);
  if (p.split > 1 && (workspace == nullptr || workspace_bytes < p.bytes)) {
    p.full = p.tiles;
    p.split = 1;
  }
  const int64_t tail = p.tiles - p.full;
  const int64_t grid = p.full + tail * p.split;
  float* partial = static_cast<float*>(p.split > 1 ? workspace : nullptr);
  k_gemm_mxfp4<<<(unsigned)grid, 256, MX_LDS_BYTES, s>>>((int)M, (int)N, (int)K, a_codes, a_scales,
                                                         b_codes, b_scales, c, ldc, accumulate,
                                                         (int)p.full, p.split, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.split == 1) return e;
  return launch_split_reduce(M, N, p, partial, nullptr, nullptr, c, 0, ldc, accumulate, s);
}

}  // namespace nvfp4
