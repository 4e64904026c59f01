// Kernel launchers shared by the C-ABI entry points (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

hipError_t launch_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                           int layout, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                           uint8_t* codes_t, uint8_t* scales_t, float* tensor_scale, float* amax,
                           hipStream_t s);

// Single-pass row-1D quantization when the tensor fits in the resident
// grid's registers (contiguous rows, stream not capturing, an exchange slot
// free); *done tells whether it ran (nothing is enqueued otherwise).
hipError_t try_quantize_row_1pass(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                  int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                                  float* tensor_scale, float* amax, hipStream_t s, bool* done);
struct GridSyncSlot;
// The per-(device, stream) exchange slot, or nullptr where none may be used.
GridSyncSlot* stream_sync_slot(hipStream_t s);
// What one single-pass launch on (current device, stream) needs: its
// exchange slot, a fresh epoch and the spin limit.  single_pass_ticket
// returns false (nothing reserved) where no single pass may run: two passes
// forced, a stream under graph capture, or no slot free on the device.
// single_pass_launched counts a launch that was enqueued with the ticket.
struct SinglePassTicket {
  GridSyncSlot* slot;
  uint32_t epoch;
  uint64_t spin;
  int dev;
};
bool single_pass_ticket(hipStream_t s, SinglePassTicket* t);
void single_pass_launched(const SinglePassTicket& t);
// 0: automatic choice of the single-pass path, 2: always two passes.
hipError_t set_quantize_passes(int passes);
// Polls a single-pass workgroup makes before it gives up waiting.
hipError_t set_sync_spin_limit(uint64_t polls);
// Single-pass launches on the current device and their workgroups that gave up.
hipError_t single_pass_stats(int64_t* launches, int64_t* give_ups);

hipError_t launch_rht_quantize(const void* x, int dt, int64_t tokens, int64_t cols, int64_t ld,
                               uint32_t sign_mask, int rnd, uint64_t seed, uint8_t* codes,
                               uint8_t* scales, float* tensor_scale, float* amax, hipStream_t s);

hipError_t launch_quantize_row_rht(const void* x, int dt, int64_t tokens, int64_t cols, int64_t ld,
                                   int row_rnd, uint64_t row_seed, uint8_t* row_codes,
                                   uint8_t* row_scales, float* row_ts, float* row_amax,
                                   uint32_t sign_mask, int rht_rnd, uint64_t rht_seed,
                                   uint8_t* rht_codes, uint8_t* rht_scales, float* rht_ts,
                                   float* rht_amax, hipStream_t s);

// c: FP32, or BF16 bits when c_bf16 is set.
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                       const uint8_t* a_scales, const float* a_ts, const uint8_t* b_codes,
                       const uint8_t* b_scales, int b_rowdiv, const float* b_ts, void* c, int c_bf16,
                       int64_t ldc, int accumulate, void* workspace, int64_t workspace_bytes,
                       hipStream_t s);

// out[r][c] = e2m1(code) * dec(scale of (r / scale_rowdiv, c / 16)) * tensor_scale,
// FP32, or BF16 bits (that FP32 value rounded to nearest even) when out_bf16.
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int scale_rowdiv,
                             const float* tensor_scale, int64_t rows, int64_t cols, void* out,
                             int out_bf16, int64_t ld_out, hipStream_t s);

hipError_t launch_mx_quantize(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                              int layout, int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                              hipStream_t s);

hipError_t launch_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                          const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                          float* c, int64_t ldc, int accumulate, void* workspace,
                          int64_t workspace_bytes, hipStream_t s);

// launch_gemm (FP32 output) with the split-tail partials in the library's
// per-device static workspace instead of a caller's buffer; it never
// allocates.  static_workspace_bytes() is that workspace's size.
hipError_t launch_gemm_static_ws(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                                 const uint8_t* a_scales, const float* a_ts,
                                 const uint8_t* b_codes, const uint8_t* b_scales, int b_rowdiv,
                                 const float* b_ts, float* c, int64_t ldc, int accumulate,
                                 hipStream_t s);
int64_t static_workspace_bytes();

// Workspace bytes launch_gemm (and launch_mx_gemm) uses for this shape on the current device
// (0: no split).
int64_t gemm_workspace_size(int64_t M, int64_t N, int64_t K);

}  // namespace nvfp4
