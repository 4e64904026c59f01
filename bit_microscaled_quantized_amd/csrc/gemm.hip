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
// (16 bytes) of row r lands in slot 8r + (c ^ ((r >> 1) & 7)).  gfx950's LDS
// serves a 16-byte read for 16 lanes per cycle (64 banks): with 128-byte rows,
// rows of equal parity share a bank half, so the 16 rows a fragment read
// touches at once need 8 distinct slots per parity -- (r >> 1) & 7 gives that
// (measured: 1.8x the read rate of c ^ (r & 7), which conflicts 2-way).
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
// of output tiles (shared L2).  The FP32 output is written with non-temporal
// stores: it is not read again by the next kernels of the step, and leaving it
// dirty in the 256 MB Infinity Cache would make them pay for its write-back.
//
// Grid tail: with one 256 x 256 tile per CU, a tile count that is not a
// multiple of the CU count leaves the last round partly idle (8192 x 5120
// output: 640 tiles = 2.5 rounds).  Given a workspace, the launcher keeps the
// whole rounds as they are and splits each of the t tiles of the last round
// into S contiguous K ranges (t * S <= CUs); those units store their raw FP32
// partial tiles in the workspace and a second kernel adds them in the fixed
// order 0 .. S-1, scales by the tensor scales and applies beta, so the result
// does not depend on scheduling.
#include <mutex>

#include "gemm_tiling.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

namespace {

constexpr int SCALE_BYTES = BM * (BKS / 16);       // 4 KB per operand
constexpr int OFF_SA = 2 * CODE_BYTES;             // A scales
constexpr int OFF_SB = 2 * CODE_BYTES + SCALE_BYTES;
constexpr int STAGE_BYTES = 2 * CODE_BYTES + 2 * SCALE_BYTES;  // 72 KB
constexpr int LDS_BYTES = 2 * STAGE_BYTES;                     // 144 KB

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

// OutT: float (FP32 output) or uint16_t (BF16 bits, rounded to nearest even
// once, after alpha and beta are applied in FP32).
template <typename OutT>
__global__ __launch_bounds__(512, 1) void k_gemm_nvfp4(
    int M, int N, int K, const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const float* __restrict__ a_ts, const uint8_t* __restrict__ b_codes,
    const uint8_t* __restrict__ b_scales, int b_rowdiv, const float* __restrict__ b_ts,
    OutT* __restrict__ c, int64_t ldc, int accumulate, int full_tiles, int split,
    float* __restrict__ partial) {
  extern __shared__ __align__(16) uint8_t lds[];

  const int KT = (K + BKS - 1) / BKS;
  const int bid = blockIdx.x;
  int id, kt0 = 0, kt1 = KT;
  float* part = nullptr;
  if (bid < full_tiles) {
    // XCD-aware order: the hardware deals workgroups round-robin over the 8
    // XCDs, so each XCD's share becomes a contiguous range of ordered tiles.
    const int G = full_tiles;
    const int xcd = bid & 7, per = G >> 3, rem = G & 7;
    id = (xcd < rem) ? xcd * (per + 1) + (bid >> 3) : rem * (per + 1) + (xcd - rem) * per + (bid >> 3);
  } else {
    // split unit u = tail tile (u / split), K part (u % split)
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
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5;
  const int lr = lane & 31;
  const int64_t kb = K / 2;   // code bytes per row (a multiple of 32)
  const int64_t ks = K / 16;  // scale bytes per row (a multiple of 4)

  // ---- stage fetch.  Code instruction j of a wave: rows r = 8(4 wave + j) +
  // l/8; lane l fills slot l%8 of its row, i.e. takes chunk
  // (l%8) ^ ((r >> 1) & 7) = (l%8) ^ (4 (j & 1) + (l/8) / 2).  Scale
  // instruction i: rows 32 wave + 16 i + l/4, lane l takes dword l%4 of the
  // row's 16 bytes.
  const int crow = lane >> 3;
  const int cchunk_e = (lane & 7) ^ (crow >> 1);        // even j
  const int cchunk_o = (lane & 7) ^ (4 + (crow >> 1));  // odd j
  const int sdw = lane & 3;
  // Per-lane 32-bit offsets of each fetch from its operand's first byte
  // (code and scale arrays are below 4 GiB, checked by the host): row start
  // plus the lane's chunk or dword.  They stay fixed over the K loop; a full
  // stage adds its wave-uniform start, kt * 128 code bytes (kt * 16 scale
  // bytes), as a scalar base, so the fetch holds 12 offset registers rather
  // than 12 64-bit row pointers.
  uint32_t o_a[4], o_b[4], o_sa[2], o_sb[2];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int r = 8 * (4 * wave + j) + crow;
    const int c16 = 16 * ((j & 1) ? cchunk_o : cchunk_e);
    o_a[j] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)kb + c16;
    o_b[j] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)kb + c16;
  }
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int r = 32 * wave + 16 * i + (lane >> 2);
    o_sa[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)ks + 4 * sdw;
    o_sb[i] = (uint32_t)(min(n0 + r, N - 1) / b_rowdiv) * (uint32_t)ks + 4 * sdw;
  }
  const uint32_t c16e = 16 * cchunk_e, c16o = 16 * cchunk_o, s4 = 4 * sdw;
  auto issue_stage = [&](int kt, uint8_t* st) {
    const uint8_t* ab = a_codes + kt * (BKS / 2);
    const uint8_t* bb = b_codes + kt * (BKS / 2);
    const uint8_t* asb = a_scales + kt * (BKS / 16);
    const uint8_t* bsb = b_scales + kt * (BKS / 16);
    // In a stage that ends past K, each in-row offset is clamped to the row's
    // last chunk (dword), so every address stays inside its row: the lane's
    // offset moves back by d (mod 2^32; the clamped offset is >= 0).
    uint32_t de = 0, dod = 0, dsc = 0;
    if ((kt + 1) * BKS > K) {
      const uint32_t ck = (uint32_t)kt * (BKS / 2), sk = (uint32_t)kt * (BKS / 16);
      de = min(ck + c16e, (uint32_t)kb - 16) - (ck + c16e);
      dod = min(ck + c16o, (uint32_t)kb - 16) - (ck + c16o);
      dsc = min(sk + s4, (uint32_t)ks - 4) - (sk + s4);
    }
    // (the empty asm keeps each offset a 32-bit register at the load, so
    // the load takes the scalar-base + 32-bit-offset form)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t oa = o_a[j] + ((j & 1) ? dod : de), ob = o_b[j] + ((j & 1) ? dod : de);
      asm volatile("" : "+v"(oa), "+v"(ob));
      load_lds16(ab + oa, st + (4 * wave + j) * 1024);
      load_lds16(bb + ob, st + OFF_B + (4 * wave + j) * 1024);
    }
#pragma unroll
    for (int i = 0; i < 2; i++) {
      uint32_t oa = o_sa[i] + dsc, ob = o_sb[i] + dsc;
      asm volatile("" : "+v"(oa), "+v"(ob));
      load_lds4(asb + oa, st + OFF_SA + (2 * wave + i) * 256);
      load_lds4(bsb + ob, st + OFF_SB + (2 * wave + i) * 256);
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
  // 8*row + ((4h + g) ^ ((lr >> 1) & 7)); its two scale bytes (blocks 2(4h + g) and
  // 2(4h + g) + 1) sit at row*16 + 2(4h + g).
  const int rowa = wm * 128 + lr;
  const int rowb = wn * 64 + lr;
  auto read_quad = [&](const uint8_t* st, int g, uint4* ca, uint4* cb, uint32_t* sa, uint32_t* sb) {
    const int sw = ((4 * h + g) ^ ((lr >> 1) & 7)) << 4;
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

  // MFMA steps s0 .. s1-1 of the quad in buffer p: per step, convert the 6
  // fragments (48 VALU) and issue 8 MFMAs; the other wave on the SIMD
  // overlaps them.  sca / scb: the quad's block scales as FP16 pairs.
  auto quad_scales = [&](int p, half2_t (&sca)[4][2], half2_t (&scb)[2][2]) {
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
  };
  auto quad_steps = [&](int p, int s0, int s1, const half2_t (&sca)[4][2], const half2_t (&scb)[2][2]) {
#pragma unroll
    for (int s = s0; s < s1; s++) {
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
  auto quad = [&](int p) {
    half2_t sca[4][2], scb[2][2];
    quad_scales(p, sca, scb);
    quad_steps(p, 0, 4, sca, scb);
  };

  // prologue: stage kt0 in buffer 0, its quad 0 read
  issue_stage(kt0, lds);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  fix_partial(kt0, lds);
  __syncthreads();
  read_quad(lds, 0, qa[0], qb[0], qsa[0], qsb[0]);

  // One stage.  cur and nxt are the two (disjoint) stage buffers; declaring
  // them restrict lets the compiler see that the fragment reads of cur do not
  // depend on the direct-to-LDS prefetch into nxt, so it does not wait for
  // that prefetch before the reads.
  auto stage = [&](int kt, const uint8_t* __restrict__ cur, uint8_t* __restrict__ nxt) {
    const bool more = kt + 1 < kt1;
    if (more) issue_stage(kt + 1, nxt);
    // quads 0..2: read the following quad of this stage while computing
    // (the reads are placed after the quad's first step, so they have three
    // steps of MFMAs to land before the next quad waits for them)
#pragma unroll
    for (int g = 0; g < 3; g++) {
      const int p = g & 1;
      half2_t sca[4][2], scb[2][2];
      quad_scales(p, sca, scb);
      quad_steps(p, 0, 1, sca, scb);
      __builtin_amdgcn_sched_barrier(8);
      read_quad(cur, g + 1, qa[p ^ 1], qb[p ^ 1], qsa[p ^ 1], qsb[p ^ 1]);
      __builtin_amdgcn_sched_barrier(8);
      quad_steps(p, 1, 4, sca, scb);
#pragma unroll
      for (int k = 0; k < 24; k++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
      }
      __builtin_amdgcn_sched_barrier(8);
    }
    // quad 3 (buffer 1): the next stage becomes visible, and its quad 0 is
    // read into buffer 0 while this stage's last quad is computed.  Every wave
    // reaches this barrier with its last reads of cur complete (quad 3 came
    // in during quad 2, and the wait covers LDS reads too), so the barrier
    // also releases cur for the prefetch the next stage issues into it.
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
  };
  for (int kt = kt0; kt < kt1; kt++) {
    uint8_t* cur = lds + ((kt - kt0) & 1) * STAGE_BYTES;
    uint8_t* nxt = lds + ((kt - kt0 + 1) & 1) * STAGE_BYTES;
    stage(kt, cur, nxt);
  }

  if (part != nullptr) {
    // raw partial tile, row-major 256 x 256 (rows / columns past M / N are
    // stored too and ignored by the reduction)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int tm = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          part[tm * BN + wn * 64 + j * 32 + lr] = acc[i][j][r];
        }
    return;
  }
  const float alpha = a_ts[0] * b_ts[0];
  // The wave tile is written one 32 x 32 MFMA tile t = 2i + j at a time.  With
  // beta = 1 the 16 old values a lane needs from tile t + 1 are loaded
  // together while tile t is stored: the compiler cannot tell the loads from
  // the stores apart (both go through c), so a load placed after a store would
  // wait for it, one round trip per element.
  float old[2][16];
  auto load_old = [&](int t, float* o) {
    const int n = n0 + wn * 64 + (t & 1) * 32 + lr;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int m = m0 + wm * 128 + (t >> 1) * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      o[r] = (m < M && n < N) ? OutElem<OutT>::load_nt(c + (int64_t)m * ldc + n) : 0.0f;
    }
  };
  if (accumulate) load_old(0, old[0]);
#pragma unroll
  for (int t = 0; t < 8; t++) {
    if (accumulate && t + 1 < 8) load_old(t + 1, old[(t + 1) & 1]);
    const int i = t >> 1, j = t & 1;
    const int n = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int m = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
      if (m < M && n < N) {
        float v = alpha * acc[i][j][r];
        if (accumulate) v += old[t & 1][r];
        OutElem<OutT>::store_nt(c + (int64_t)m * ldc + n, v);
      }
    }
  }
}

// Sum of the S partial tiles of each split tail tile in the order 0 .. S-1,
// then C = alpha * sum (+ C).  Block (x, t): tail tile t, rows 4x .. 4x + 3;
// thread: one row, four consecutive columns.
template <typename OutT>
__global__ __launch_bounds__(256) void k_gemm_split_reduce(int M, int N, int full_tiles, int split,
                                                           const float* __restrict__ partial,
                                                           const float* __restrict__ a_ts,
                                                           const float* __restrict__ b_ts,
                                                           OutT* __restrict__ c, int64_t ldc,
                                                           int accumulate) {
  const int t = blockIdx.y;
  int pm, pn;
  tile_of(full_tiles + t, (M + BM - 1) / BM, (N + BN - 1) / BN, pm, pn);
  const int e = blockIdx.x * 256 + threadIdx.x;  // float4 index inside the tile
  const int r = e / (BN / 4), c4 = (e % (BN / 4)) * 4;
  const int m = pm * BM + r, n = pn * BN + c4;
  if (m >= M || n >= N) return;  // N is a multiple of 16: a float4 is all in or all out
  const float4* src = reinterpret_cast<const float4*>(partial + (int64_t)t * split * (BM * BN)) + e;
  float4 v = src[0];
  for (int q = 1; q < split; q++) {
    const float4 w = src[(int64_t)q * (BM * BN / 4)];
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  const float alpha = a_ts != nullptr ? a_ts[0] * b_ts[0] : 1.0f;  // null: no tensor scales (MXFP4)
  float4 o = make_float4(alpha * v.x, alpha * v.y, alpha * v.z, alpha * v.w);
  OutT* dst = c + (int64_t)m * ldc + n;
  if constexpr (sizeof(OutT) == 4) {
    float4* d4 = reinterpret_cast<float4*>(dst);
    if (accumulate) {
      const float4 old = *d4;
      o.x += old.x; o.y += old.y; o.z += old.z; o.w += old.w;
    }
    __builtin_nontemporal_store(o.x, &d4->x);
    __builtin_nontemporal_store(o.y, &d4->y);
    __builtin_nontemporal_store(o.z, &d4->z);
    __builtin_nontemporal_store(o.w, &d4->w);
  } else {
    uint2* d2 = reinterpret_cast<uint2*>(dst);  // four BF16 values
    if (accumulate) {
      const uint2 old = *d2;
      o.x += bf16lo(old.x); o.y += bf16hi(old.x); o.z += bf16lo(old.y); o.w += bf16hi(old.y);
    }
    const uint32_t lo = bf16_rne(o.x) | (bf16_rne(o.y) << 16);
    const uint32_t hi = bf16_rne(o.z) | (bf16_rne(o.w) << 16);
    __builtin_nontemporal_store(lo, &d2->x);
    __builtin_nontemporal_store(hi, &d2->y);
  }
}

namespace {

constexpr int kMaxDevices = 64;

// Compute units of the current device (cached per device, no allocation).
int device_cus() {
  static std::mutex mu;
  static int cache[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cache[dev] = n;
  }
  return cache[dev];
}

// Split-tail workspace of the allocation-free entry point, one copy per
// device for the life of the process.  The split plan fills at most one round
// of 256 x 256 FP32 partial tiles, 256 KiB per compute unit: 64 MiB holds the
// plan of any shape on a 256-CU MI355X.  Every call on a device shares its
// copy; the GEMM writes each partial tile whole before the reduction reads
// it, so nothing needs clearing, but calls that overlap on one device race.
constexpr int64_t kStaticWorkspaceBytes = int64_t(64) << 20;
__device__ __align__(256) float scratch[kStaticWorkspaceBytes / 4];

// Device address of the current device's `scratch`, looked up once per
// device (the host-side name is not a device address).
hipError_t static_workspace(void** ptr) {
  static std::mutex mu;
  static void* cache[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    cache[dev] = p;
  }
  *ptr = cache[dev];
  return hipSuccess;
}

}  // namespace

// Tail tiles t = tiles mod CUs; split S = min(CUs / t, KT / 4, 16) when that
// is at least 2, so the t * S units fill at most one round and each part
// keeps at least four K stages.
SplitPlan plan_split(int64_t M, int64_t N, int64_t K) {
  SplitPlan p;
  p.tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  p.full = p.tiles;
  const int cus = device_cus();
  if (cus <= 0) return p;
  const int64_t t = p.tiles % cus;
  const int64_t kt = (K + BKS - 1) / BKS;
  if (t == 0) return p;
  const int64_t s = std::min<int64_t>(std::min<int64_t>(cus / t, kt / 4), 16);
  if (s < 2) return p;
  p.full = p.tiles - t;
  p.split = (int)s;
  p.bytes = t * s * (int64_t)(BM * BN) * (int64_t)sizeof(float);
  return p;
}

hipError_t launch_split_reduce(int64_t M, int64_t N, const SplitPlan& p, const float* partial,
                               const float* a_ts, const float* b_ts, void* c, int c_bf16,
                               int64_t ldc, int accumulate, hipStream_t s) {
  const dim3 grid(BM * BN / 4 / 256, (unsigned)(p.tiles - p.full));
  if (c_bf16)
    k_gemm_split_reduce<uint16_t><<<grid, 256, 0, s>>>((int)M, (int)N, (int)p.full, p.split, partial,
                                                       a_ts, b_ts, static_cast<uint16_t*>(c), ldc,
                                                       accumulate);
  else
    k_gemm_split_reduce<float><<<grid, 256, 0, s>>>((int)M, (int)N, (int)p.full, p.split, partial,
                                                    a_ts, b_ts, static_cast<float*>(c), ldc, accumulate);
  return hipGetLastError();
}

int64_t gemm_workspace_size(int64_t M, int64_t N, int64_t K) { return plan_split(M, N, K).bytes; }

namespace {

template <typename OutT>
hipError_t launch_gemm_t(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                         const uint8_t* a_scales, const float* a_ts, const uint8_t* b_codes,
                         const uint8_t* b_scales, int b_rowdiv, const float* b_ts, OutT* c,
                         int64_t ldc, int accumulate, void* workspace, int64_t workspace_bytes,
                         hipStream_t s) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_gemm_nvfp4<OutT>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, LDS_BYTES);
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
  k_gemm_nvfp4<OutT><<<(unsigned)grid, 512, LDS_BYTES, s>>>(
      (int)M, (int)N, (int)K, a_codes, a_scales, a_ts, b_codes, b_scales, b_rowdiv, b_ts, c, ldc,
      accumulate, (int)p.full, p.split, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.split == 1) return e;
  return launch_split_reduce(M, N, p, partial, a_ts, b_ts, c, sizeof(OutT) == 2, ldc, accumulate, s);
}

}  // namespace

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_ts, const uint8_t* b_codes,
                       const uint8_t* b_scales, int b_rowdiv, const float* b_ts, void* c, int c_bf16,
                       int64_t ldc, int accumulate, void* workspace, int64_t workspace_bytes,
                       hipStream_t s) {
  if (c_bf16)
    return launch_gemm_t(M, N, K, a_codes, a_scales, a_ts, b_codes, b_scales, b_rowdiv, b_ts,
                         static_cast<uint16_t*>(c), ldc, accumulate, workspace, workspace_bytes, s);
  return launch_gemm_t(M, N, K, a_codes, a_scales, a_ts, b_codes, b_scales, b_rowdiv, b_ts,
                       static_cast<float*>(c), ldc, accumulate, workspace, workspace_bytes, s);
}

int64_t static_workspace_bytes() { return kStaticWorkspaceBytes; }

hipError_t launch_gemm_static_ws(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                                 const uint8_t* a_scales, const float* a_ts,
                                 const uint8_t* b_codes, const uint8_t* b_scales, int b_rowdiv,
                                 const float* b_ts, float* c, int64_t ldc, int accumulate,
                                 hipStream_t s) {
  void* ws = nullptr;
  hipError_t e = static_workspace(&ws);
  if (e != hipSuccess) return e;
  return launch_gemm_t(M, N, K, a_codes, a_scales, a_ts, b_codes, b_scales, b_rowdiv, b_ts, c, ldc,
                       accumulate, ws, kStaticWorkspaceBytes, s);
}

}  // namespace nvfp4
