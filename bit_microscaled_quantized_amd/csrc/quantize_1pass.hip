// Single-pass row-1D NVFP4 quantization for tensors that fit on chip.
//
// The method needs the tensor amax before any element can be encoded
// ("Pretraining Large Language Models with NVFP4", gist.science summary,
// Resumo tecnico, 2. Metodologia Proposta, "Escala em Dois Niveis": the FP32
// tensor scale maps the tensor maximum onto the FP4 x E4M3 range).  The
// two-pass path reads the input twice for that.  Here one launch whose
// workgroups are all resident reads the whole tensor into registers once:
//   phase 1: every lane loads its blocks of 16 elements (all loads issued
//            first) and takes each block's maximum; the workgroup's maximum
//            goes to the device-wide exchange of grid_sync.hpp;
//   phase 2: once the tensor amax is published, each lane encodes its blocks
//            from registers (the arithmetic of the two-pass row cast, so the
//            codes are identical) and stores codes and scales.
// The grid never exceeds the number of workgroups that fit on the device at
// once, so normally all arrive within microseconds.  The wait is bounded all
// the same: a workgroup that waits too long (its grid partly displaced by
// other streams' kernels) gives up and leaves its blocks to the publisher
// (the last workgroup to arrive), which encodes them from memory once its
// own are done, so the outputs are always complete.  No workgroup waits for
// the others to finish.  A cooperative launch would give co-residency
// outright but costs ~14 us per call on this runtime, most of the single
// pass's gain.
//
// Layout: contiguous rows only (ld == cols), seen as one sequence of 16-element
// blocks; wave v of the grid holds blocks (v * rounds + r) * 64 + lane, so
// each load and store instruction covers 64 consecutive blocks.  codes
// [rows][cols/2], scales [rows][cols/16], as the row cast.
#include <mutex>

#include "grid_sync.hpp"
#include "sync_ops.hpp"
#include "nvfp4_device.hpp"
#include "nvfp4_launch.hpp"

namespace nvfp4 {

namespace {

// Exchange slots, one per (device, stream) in use: calls on one stream run in
// order, so a slot is never used by two launches at once.  Each device holds
// its own copy of the array.
constexpr int kSyncSlots = 64;
__device__ __align__(256) GridSyncSlot sync_slots[kSyncSlots];

// One 16-element block as loaded.
template <typename T>
struct Blk;
template <>
struct Blk<uint16_t> {
  uint4 w[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    w[0] = reinterpret_cast<const uint4*>(p)[0];
    w[1] = reinterpret_cast<const uint4*>(p)[1];
  }
  // maximum |x| as FP32 bits (exact: a bf16 value)
  __device__ __forceinline__ uint32_t absmax_bits() const {
    uint32_t m = 0u;
#pragma unroll
    for (int h = 0; h < 2; h++) {
      m = absmax_bf16x2(m, w[h].x);
      m = absmax_bf16x2(m, w[h].y);
      m = absmax_bf16x2(m, w[h].z);
      m = absmax_bf16x2(m, w[h].w);
    }
    return m << 16;
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
struct Blk<float> {
  float4 w[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int q = 0; q < 4; q++) w[q] = reinterpret_cast<const float4*>(p)[q];
  }
  __device__ __forceinline__ uint32_t absmax_bits() const {
    uint32_t m = 0u;
#pragma unroll
    for (int q = 0; q < 4; q++) {
      m = max(m, __float_as_uint(w[q].x) & 0x7FFFFFFFu);
      m = max(m, __float_as_uint(w[q].y) & 0x7FFFFFFFu);
      m = max(m, __float_as_uint(w[q].z) & 0x7FFFFFFFu);
      m = max(m, __float_as_uint(w[q].w) & 0x7FFFFFFFu);
    }
    return m;
  }
  __device__ __forceinline__ void get(float* v) const {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      v[4 * q + 0] = w[q].x; v[4 * q + 1] = w[q].y; v[4 * q + 2] = w[q].z; v[4 * q + 3] = w[q].w;
    }
  }
};

// Encode 16 scaled values (RNE in hardware; SR with the pcg bits of output
// elements 2 pair0 .. 2 pair0 + 15, pair0 a multiple of 8).
template <int RND>
__device__ __forceinline__ uint2 encode_blk(const float* v, uint32_t key, uint32_t pair0) {
  if constexpr (RND == 0) {
    return make_uint2(pack8_rne(v), pack8_rne(v + 8));
  } else {
    uint32_t h[8];
    pcg8(key, pair0, h);
    return make_uint2(sr_pack8(v, h), sr_pack8(v + 8, h + 4));
  }
}

// Block r of lane `lane` in wave v of the grid (rounds blocks per lane).
__device__ __forceinline__ uint32_t block_of(uint32_t v, uint32_t rounds, uint32_t r, uint32_t lane) {
  return (v * rounds + r) * 64u + lane;
}

// Scale and encode one block whose values and maximum are at hand; store its
// codes and scale.
template <typename T, int RND>
__device__ __forceinline__ void encode_store(const Blk<T>& blk, uint32_t bmax, uint32_t b, float s_enc,
                                             const float* rtab, uint32_t key, uint8_t* codes,
                                             uint8_t* scales) {
  uint32_t e_b;
  float r_b;
  block_scale(__uint_as_float(bmax), s_enc, rtab, e_b, r_b);
  float v[16];
  blk.get(v);
#pragma unroll
  for (int e = 0; e < 16; e++) v[e] *= r_b;
  st_nt(codes + (size_t)b * 8, encode_blk<RND>(v, key, b * 8u));
  st_nt8(scales + b, (uint8_t)e_b);
}

// NB: blocks per lane (compile time); rounds <= NB of them are used.
template <typename T, int RND, int NB>
__global__ __launch_bounds__(256, 2) void k_quant_row_1pass(
    const T* __restrict__ x, uint32_t nblocks, uint32_t rounds, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, float* __restrict__ tensor_scale, float* __restrict__ amax_out,
    uint32_t key, GridSyncSlot* slot, uint32_t epoch, uint64_t spin_limit) {
  __shared__ float rtab[128];
  __shared__ uint32_t wave_max[4];
  __shared__ uint32_t sh_amax, sh_role, sh_n;
  const uint32_t G = gridDim.x;
  const uint32_t tid = threadIdx.x, lane = tid & 63u;
  const uint32_t wave = blockIdx.x * 4u + (tid >> 6);

  // phase 1: all loads first, then the block maxima
  Blk<T> blk[NB];
#pragma unroll
  for (int r = 0; r < NB; r++) {
    const uint32_t b = block_of(wave, rounds, r, lane);
    if (r < (int)rounds && b < nblocks) blk[r].load(x + (size_t)b * 16);
  }
  uint32_t bmax[NB];
  uint32_t m = 0u;
#pragma unroll
  for (int r = 0; r < NB; r++) {
    const uint32_t b = block_of(wave, rounds, r, lane);
    bmax[r] = (r < (int)rounds && b < nblocks) ? blk[r].absmax_bits() : 0u;
    m = max(m, bmax[r]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor(m, off));
  if (lane == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    const uint32_t wm = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
    uint32_t bits = 0u, n = 0u;
    sh_role = grid_arrive_wait<DeviceOps>(slot, G, blockIdx.x, wm, epoch, spin_limit, &bits, &n);
    sh_amax = bits;
    sh_n = n;
  }
  __syncthreads();
  // a workgroup that gave up leaves its blocks to the publisher
  if (sh_role == kGridGaveUp) return;

  // phase 2: encode from registers
  const float amax_t = __uint_as_float(sh_amax);
  const float s_enc = encode_scale(amax_t);
  fill_scale_table(rtab, s_enc);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < NB; r++) {
    const uint32_t b = block_of(wave, rounds, r, lane);
    if (r < (int)rounds && b < nblocks)
      encode_store<T, RND>(blk[r], bmax[r], b, s_enc, rtab, key, codes, scales);
  }
  if (sh_role != kGridPublisher) return;

  // the publisher: the tensor outputs, and the blocks of the workgroups that
  // gave up, read again from memory
  if (tid == 0) {
    tensor_scale[0] = 1.0f / s_enc;
    amax_out[0] = amax_t;
  }
  for (uint32_t i = 0; i < sh_n; i++) {
    __shared__ uint32_t sh_w;
    if (tid == 0) sh_w = grid_recovered<DeviceOps>(slot, i, uint64_t(1) << 22);
    __syncthreads();
    const uint32_t w = sh_w;
    __syncthreads();
    if (w >= G) continue;  // never stored (cannot happen: the entry follows its swap)
    for (uint32_t r = 0; r < rounds; r++) {
      const uint32_t b = block_of(w * 4u + (tid >> 6), rounds, r, lane);
      if (b < nblocks) {
        Blk<T> one;
        one.load(x + (size_t)b * 16);
        encode_store<T, RND>(one, one.absmax_bits(), b, s_enc, rtab, key, codes, scales);
      }
    }
  }
}

// Blocks per lane of the two instances: 20 for bf16 (160 data VGPRs at two
// waves per SIMD, the 84 MB of an 8192 x 5120 bf16 tensor on 256 CUs), 10 for
// FP32.
template <typename T>
constexpr int blocks_per_lane() {
  return sizeof(T) == 2 ? 20 : 10;
}

struct Resident {
  int cus = 0;
  int per_cu[2][2] = {};  // [fp32][SR] resident workgroups per CU, 0 = not supported
};

constexpr int kMaxDevices = 64;

template <typename T, int RND>
const void* kernel_ptr() {
  return reinterpret_cast<const void*>(&k_quant_row_1pass<T, RND, blocks_per_lane<T>()>);
}

std::mutex g_mu;
uint32_t g_epoch[kMaxDevices][kSyncSlots] = {};
Resident g_res[kMaxDevices];
bool g_res_done[kMaxDevices] = {};
GridSyncSlot* g_slots[kMaxDevices] = {};
void* g_slot_stream[kMaxDevices][kSyncSlots] = {};
int g_slot_used[kMaxDevices] = {};
int g_passes = 0;  // 0: automatic, 2: always the two-pass path
int64_t g_launches[kMaxDevices] = {};  // single-pass launches enqueued per device
uint64_t g_spin_limit = uint64_t(1) << 14;

// Per-device set-up under g_mu: residency of the four instances, and the
// device address of this device's slot array (zeroed once).
bool device_setup(int dev) {
  if (g_res_done[dev]) return g_slots[dev] != nullptr;
  g_res_done[dev] = true;
  Resident r;
  if (hipDeviceGetAttribute(&r.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
  const void* k[2][2] = {{kernel_ptr<uint16_t, 0>(), kernel_ptr<uint16_t, 1>()},
                         {kernel_ptr<float, 0>(), kernel_ptr<float, 1>()}};
  for (int f = 0; f < 2; f++)
    for (int s = 0; s < 2; s++) {
      int n = 0;
      if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k[f][s], 256, 0) != hipSuccess) n = 0;
      r.per_cu[f][s] = n;
    }
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(sync_slots)) != hipSuccess) return false;
  if (hipMemset(p, 0, sizeof(GridSyncSlot) * kSyncSlots) != hipSuccess) return false;
  g_res[dev] = r;
  g_slots[dev] = static_cast<GridSyncSlot*>(p);
  return true;
}

// The slot of (device, stream), assigned on first use; -1 when all are taken.
int slot_of(int dev, void* stream) {
  for (int i = 0; i < g_slot_used[dev]; i++)
    if (g_slot_stream[dev][i] == stream) return i;
  if (g_slot_used[dev] == kSyncSlots) return -1;
  g_slot_stream[dev][g_slot_used[dev]] = stream;
  return g_slot_used[dev]++;
}

}  // namespace

// The exchange slot of (current device, stream) for the amax passes of the
// two-pass path, or nullptr (stream under graph capture, set-up failed, or
// all slots of the device taken by other streams).
GridSyncSlot* stream_sync_slot(hipStream_t s) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!device_setup(dev)) return nullptr;
  const int i = slot_of(dev, s);
  return i < 0 ? nullptr : g_slots[dev] + i;
}

bool single_pass_ticket(hipStream_t s, SinglePassTicket* t) {
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return false;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_passes == 2 || !device_setup(dev)) return false;
  const int si = slot_of(dev, s);
  if (si < 0) return false;
  if (++g_epoch[dev][si] == 0u) g_epoch[dev][si] = 1u;  // 0 is the zeroed slot's value
  t->slot = g_slots[dev] + si;
  t->epoch = g_epoch[dev][si];
  t->spin = g_spin_limit;
  t->dev = dev;
  return true;
}

void single_pass_launched(const SinglePassTicket& t) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_launches[t.dev]++;
}

// Try the single-pass row-1D quantization; *done = false (and nothing
// enqueued) when it does not apply: strided rows, a tensor larger than the
// resident grid holds, a stream under graph capture, or all exchange slots of
// the device taken by other streams.
hipError_t try_quantize_row_1pass(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld,
                                  int rnd, uint64_t seed, uint8_t* codes, uint8_t* scales,
                                  float* tensor_scale, float* amax, hipStream_t s, bool* done) {
  *done = false;
  if (ld != cols) return hipSuccess;
  // before device_setup: its first call on a device clears the slots with a
  // synchronous memset, which a stream under capture must not see
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone)
    return hipSuccess;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipSuccess;
  int per_cu = 0, cus = 0;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (!device_setup(dev)) return hipSuccess;
    per_cu = g_res[dev].per_cu[dt == 0 ? 0 : 1][rnd];
    cus = g_res[dev].cus;
  }
  if (per_cu < 1) return hipSuccess;
  const int NB = dt == 0 ? blocks_per_lane<uint16_t>() : blocks_per_lane<float>();
  const int64_t nblocks = rows * cols / 16;
  const int64_t lanes_needed = (nblocks + NB - 1) / NB;
  const int64_t max_grid = std::min<int64_t>((int64_t)per_cu * cus, kSyncMaxGrid);
  int64_t grid = (lanes_needed + 255) / 256;
  if (grid > max_grid) return hipSuccess;  // does not fit on chip: two passes
  // spread over every resident workgroup (more memory parallelism), at least
  // one block per lane
  grid = std::min<int64_t>(max_grid, std::max<int64_t>(grid, (nblocks + 255) / 256));
  const uint32_t rounds = (uint32_t)((nblocks + grid * 256 - 1) / (grid * 256));
  const uint32_t key = sr_key(seed);
  SinglePassTicket tk;
  if (!single_pass_ticket(s, &tk)) return hipSuccess;
  GridSyncSlot* slot = tk.slot;
  const uint32_t epoch = tk.epoch;
  const uint64_t spin = tk.spin;
  const uint32_t nb32 = (uint32_t)nblocks;
  if (dt == 0) {
    if (rnd == 0)
      k_quant_row_1pass<uint16_t, 0, blocks_per_lane<uint16_t>()><<<(unsigned)grid, 256, 0, s>>>(
          static_cast<const uint16_t*>(x), nb32, rounds, codes, scales, tensor_scale, amax, key, slot,
          epoch, spin);
    else
      k_quant_row_1pass<uint16_t, 1, blocks_per_lane<uint16_t>()><<<(unsigned)grid, 256, 0, s>>>(
          static_cast<const uint16_t*>(x), nb32, rounds, codes, scales, tensor_scale, amax, key, slot,
          epoch, spin);
  } else {
    if (rnd == 0)
      k_quant_row_1pass<float, 0, blocks_per_lane<float>()><<<(unsigned)grid, 256, 0, s>>>(
          static_cast<const float*>(x), nb32, rounds, codes, scales, tensor_scale, amax, key, slot,
          epoch, spin);
    else
      k_quant_row_1pass<float, 1, blocks_per_lane<float>()><<<(unsigned)grid, 256, 0, s>>>(
          static_cast<const float*>(x), nb32, rounds, codes, scales, tensor_scale, amax, key, slot,
          epoch, spin);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  *done = true;
  single_pass_launched(tk);
  return hipSuccess;
}

hipError_t set_quantize_passes(int passes) {
  if (passes != 0 && passes != 2) return hipErrorInvalidValue;
  std::lock_guard<std::mutex> lock(g_mu);
  g_passes = passes;
  return hipSuccess;
}

hipError_t set_sync_spin_limit(uint64_t polls) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_spin_limit = polls;
  return hipSuccess;
}

// Single-pass launches enqueued on the current device, and their workgroups
// that gave up waiting, summed over all slots (the caller synchronizes first).
hipError_t single_pass_stats(int64_t* launches, int64_t* count) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  GridSyncSlot* p = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    *launches = g_launches[dev];
    if (!device_setup(dev)) {
      *count = 0;
      return hipSuccess;
    }
    p = g_slots[dev];
  }
  int64_t n = 0;
  for (int i = 0; i < kSyncSlots; i++) {
    uint32_t v = 0;
    e = hipMemcpy(&v, &p[i].gave_ups, sizeof(v), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return e;
    n += v;
  }
  *count = n;
  return hipSuccess;
}

}  // namespace nvfp4
