// Tiling shared by the NVFP4 and MXFP4 GEMM kernels: 256 x 256 output tiles,
// stages of 256 K-elements whose packed FP4 codes (128 bytes per row) are
// fetched straight into LDS, the grouped tile order, and the split of the
// last, partial round of tiles over K (partial tiles in a workspace, summed
// in a fixed order by a second kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

namespace {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BKS = 256;                    // K elements per stage
constexpr int CODE_BYTES = BM * (BKS / 2);  // 32 KB of codes per operand and stage
constexpr int OFF_B = CODE_BYTES;           // B codes follow A codes in a stage

typedef __attribute__((address_space(1))) void gvoid;
typedef __attribute__((address_space(3))) void lvoid;

// Each lane's `size` bytes at g land at l + lane * size (l wave-uniform).
__device__ __forceinline__ void load_lds16(const uint8_t* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((gvoid*)g, (lvoid*)l, 16, 0, 0);
}
__device__ __forceinline__ void load_lds4(const uint8_t* g, uint8_t* l) {
  __builtin_amdgcn_global_load_lds((gvoid*)g, (lvoid*)l, 4, 0, 0);
}

// Output tile of ordered tile index id: tiles are walked in groups of GROUP
// tile rows, column by column inside a group.
constexpr int GROUP = 8;
__device__ __forceinline__ void tile_of(int id, int num_m, int num_n, int& pm, int& pn) {
  const int width = GROUP * num_n;
  const int first_m = (id / width) * GROUP;
  const int gsz = min(num_m - first_m, GROUP);
  pm = first_m + (id % width) % gsz;
  pn = (id % width) / gsz;
}

}  // namespace

struct SplitPlan {
  int64_t tiles = 0;
  int64_t full = 0;   // tiles computed whole
  int split = 1;      // K parts per tail tile (1: no split)
  int64_t bytes = 0;  // workspace bytes for the partial tiles
};

// Split of the tail tiles of an M x N x K GEMM on the current device.
SplitPlan plan_split(int64_t M, int64_t N, int64_t K);

// C = alpha * (sum of the p.split partial tiles of each tail tile) (+ C),
// alpha = a_ts[0] * b_ts[0], or 1 when a_ts is null; c is FP32, or BF16 bits
// when c_bf16 is set.
hipError_t launch_split_reduce(int64_t M, int64_t N, const SplitPlan& p, const float* partial,
                               const float* a_ts, const float* b_ts, void* c, int c_bf16,
                               int64_t ldc, int accumulate, hipStream_t s);

}  // namespace nvfp4
