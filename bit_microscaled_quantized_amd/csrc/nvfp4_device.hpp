// Device-side NVFP4 helpers for gfx950.
//
// Format and scale rule (see include/nvfp4.h for the full statement):
//   "Pretraining Large Language Models with NVFP4" (gist.science summary),
//   Resumo tecnico, 2. Metodologia Proposta, "Formato NVFP4": 16-element
//   blocks, E4M3 block scale, FP32 tensor scale.  E2M1 / E4M3 encodings per
//   the OCP MX v1.0 and OCP OFP8 specifications.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr float kFltMax = 3.402823466e+38f;

// S_enc from the tensor amax: 2688 / amax (2688 = 6 * 448, the largest
// E2M1 x E4M3 product), clamped to FLT_MAX, 1 for an all-zero tensor.
__device__ __forceinline__ float encode_scale(float amax_t) {
  if (!(amax_t > 0.0f)) return 1.0f;
  return fminf(2688.0f / amax_t, kFltMax);
}

// E4M3 code of sb >= 0: nearest finite value, ties to the even code.  The
// gfx950 conversion to OCP E4M3 does it in one instruction: it equals the
// nearest-even search (subnormal codes k * 2^-9 included) on every FP32
// input up to 464, the rounding boundary above 448, and gives NaN beyond.
// Inputs stay below 449 here: sb is RN(RN(amax_b / 6) * S_enc) with
// amax_b <= amax_t and S_enc <= 2688 / amax_t.  The second element converted
// is 0 and the upper half word is the zero passed in, so the result is the
// code itself.
__device__ __forceinline__ uint32_t e4m3_encode(float sb) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sb, 0.0f, 0, false);
}

// Value of a finite non-negative E4M3 code.
__device__ __forceinline__ float e4m3_decode(uint32_t e) {
  if (e < 8u) return (float)e * 0.001953125f;
  return __uint_as_float((e << 20) + (120u << 23));
}

// Multiplier mapping a block onto the E2M1 grid: S_enc / dec(e_b), 0 for an
// empty scale, clamped to FLT_MAX so that v = y * r_b is never NaN.
__device__ __forceinline__ float element_scale(uint32_t e_b, float s_enc) {
  if (e_b == 0u) return 0.0f;
  return fminf(s_enc / e4m3_decode(e_b), kFltMax);
}

// x / 6, correctly rounded.  For x >= 2^-100 the product with RN(1/6) plus one
// FMA correction of the exact residual is correctly rounded (checked against
// the IEEE division on every such FP32 value); below, where the quotient can
// be subnormal and that shortcut is not, the division itself runs.
__device__ __forceinline__ float div6(float x) {
  if (__builtin_expect(x < 0x1p-100f, 0)) return x / 6.0f;
  const float c = 0x1.555556p-3f;  // RN(1/6)
  const float q0 = x * c;
  return __builtin_fmaf(__builtin_fmaf(-q0, 6.0f, x), c, q0);
}

// Per-workgroup table of element_scale(e, s_enc) for every code e < 128, so a
// block needs one LDS read instead of a division.  Threads 0..127 fill it;
// the caller synchronizes before the first lookup.
__device__ __forceinline__ void fill_scale_table(float* tab, float s_enc) {
  if (threadIdx.x < 128) tab[threadIdx.x] = element_scale(threadIdx.x, s_enc);
}

// Block scale code and element multiplier from a block amax.
__device__ __forceinline__ void block_scale(float amax_b, float s_enc, const float* tab, uint32_t& e_b,
                                            float& r_b) {
  const float t = div6(amax_b);
  const float sb = t * s_enc;
  e_b = e4m3_encode(sb);
  r_b = tab[e_b];
}

// Two values to two E2M1 codes, round-to-nearest-even with saturation, placed
// in byte `sel` of `old` (v0 in the low nibble).  The gfx950 conversion with
// scale 1.0 was checked against the nearest-even rule on every FP32 value.
template <int sel>
__device__ __forceinline__ uint32_t cvt_rne_pk(uint32_t old, float v0, float v1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, v0, v1, 1.0f, sel);
}

// Pack eight scaled values into eight E2M1 codes (RNE), element 0 in the low
// nibble of byte 0.
__device__ __forceinline__ uint32_t pack8_rne(const float* v) {
  uint32_t w = 0u;
  w = cvt_rne_pk<0>(w, v[0], v[1]);
  w = cvt_rne_pk<1>(w, v[2], v[3]);
  w = cvt_rne_pk<2>(w, v[4], v[5]);
  w = cvt_rne_pk<3>(w, v[6], v[7]);
  return w;
}

// pcg hash (Jarzynski & Olano, "Hash Functions for GPU Rendering", JCGT 2020).
__device__ __forceinline__ uint32_t pcg_tail(uint32_t state) {
  const uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
  return (word >> 22u) ^ word;
}

// pcg(key ^ (pair0 + p)) for p = 0..7, pair0 a multiple of 8.  The xor then
// only touches the low three bits, so the pcg input is
// ((key ^ pair0) & ~7) + ((key & 7) ^ p) and its state
// ((key ^ pair0) & ~7) * C1 + (((key & 7) ^ p) * C1 + C2): one multiply for
// the eight pairs, the second term being uniform across the wave.
__device__ __forceinline__ void pcg8(uint32_t key, uint32_t pair0, uint32_t* h) {
  uint32_t base = ((key ^ pair0) & ~7u) * 747796405u;
  asm volatile("" : "+v"(base));  // keep the shared product: one multiply, eight adds
#pragma unroll
  for (int p = 0; p < 8; p++)
    h[p] = pcg_tail(base + ((((key & 7u) ^ (uint32_t)p) * 747796405u) + 2891336453u));
}

// pcg(key ^ (pair0 + p)) for p = 0..3, pair0 a multiple of 4 (the same
// shared-multiply form as pcg8, over the two low bits).
__device__ __forceinline__ void pcg4(uint32_t key, uint32_t pair0, uint32_t* h) {
  uint32_t base = ((key ^ pair0) & ~3u) * 747796405u;
  asm volatile("" : "+v"(base));
#pragma unroll
  for (int p = 0; p < 4; p++)
    h[p] = pcg_tail(base + ((((key & 3u) ^ (uint32_t)p) * 747796405u) + 2891336453u));
}

__host__ __device__ __forceinline__ uint32_t pcg_host(uint32_t v) {
  uint32_t state = v * 747796405u + 2891336453u;
  uint32_t word = ((state >> ((state >> 28u) + 4u)) ^ state) * 277803737u;
  return (word >> 22u) ^ word;
}

// Stochastic rounding of scaled values to E2M1 codes: with a = min(|v|, 6),
// lo the largest E2M1 magnitude <= a and hi the next one, round up iff
// r16 < frac * 2^16, frac = (a - lo) / (hi - lo) exact (r16 the element's 16
// random bits), sign kept.  It runs on gfx950's v_cvt_scalef32_sr_pk_fp4_f32,
// whose rule was measured on the device: sign-magnitude; the input is divided
// by the scale operand's power of two; with F the fraction of the quotient's
// magnitude truncated to 22 bits, floor(frac * 2^22), element 0 of the pair
// rounds up iff F + R[31:10] >= 2^22 and element 1 iff F + R[30:9] >= 2^22 (R
// the 32-bit random operand); magnitudes >= 6 give code 7.  Two adjustments
// turn that into the rule above exactly:
//   * F must count as ceil(frac * 2^22).  For a >= 1, a is a multiple of
//     2^-23 and frac * 2^22 = (a - lo) * 2^22 / step an integer (steps 1/2,
//     1, 2), so F is exact.  Below 1 the step is 1/2 and frac * 2^22 =
//     (a - lo) * 2^23: rounding |v| up to a multiple of 2^-23 first
//     (sr_hw_input; lo is on that grid) turns the truncation into the
//     ceiling, and leaves every |v| >= 1 unchanged;
//   * r16 < frac * 2^16 is 64 r16 < ceil(frac * 2^22), i.e.
//     F + (2^22 - 1 - 64 r16) >= 2^22, so the element's field must hold
//     2^22 - 1 - 64 r16: R = ~(r16 << 16) for element 0 (low 10 bits free) and
//     (~r16 << 15) | 0x7FFF for element 1 (low 9 bits free).
// The rounded-up input goes in as ceil(|v| * 2^23) with v's sign and the
// scale operand 2^23, which the conversion divides out exactly.
// The two elements of a pair draw independent bits, so each pair goes through
// two conversions, one correct in its low nibble (element 0) and one in its
// high nibble (element 1), merged by one bit select per 8 codes.

// ceil(|v| * 2^23) with v's sign, exact: every scaled value has |v| < 10 (a
// block's maximum maps to at most 6 * (1 + 2^-4) through a normal E4M3 scale
// and to at most 9 through a subnormal one; the FLT_MAX clamps only shrink
// it).
__device__ __forceinline__ float sr_hw_input(float v) {
  const float t = __builtin_ceilf(__builtin_fabsf(v) * 8388608.0f);
  return __builtin_copysignf(t, v);
}

// One SR conversion (scale 2^23) into byte `sel` of d, the other bytes of d
// kept.  Written as inline asm with d read-write: the compiler's builtin for
// this instruction does not tie its `old` operand to the destination, so the
// kept bytes would be whatever the destination register held.  The first
// conversion into a word (FIRST) writes byte 0 and leaves bytes that later
// conversions overwrite, so its destination needs no initial value.  The
// scale is an SGPR operand (this encoding takes no 32-bit literal).
template <int sel, bool FIRST = false>
__device__ __forceinline__ void cvt_sr_pk(uint32_t& d, double x, uint32_t r) {
  const float s = 8388608.0f;  // 2^23
  if constexpr (FIRST) {
    static_assert(sel == 0, "only the byte-0 conversion starts a word");
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "=v"(d) : "v"(x), "v"(r), "s"(s));
  } else if constexpr (sel == 0) {
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" : "+v"(d) : "v"(x), "v"(r), "s"(s));
  } else if constexpr (sel == 1) {
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,0]" : "+v"(d) : "v"(x), "v"(r), "s"(s));
  } else if constexpr (sel == 2) {
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,0,1]" : "+v"(d) : "v"(x), "v"(r), "s"(s));
  } else {
    asm volatile("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3 op_sel:[0,0,1,1]" : "+v"(d) : "v"(x), "v"(r), "s"(s));
  }
}

template <int sel>
__device__ __forceinline__ void sr_pk(uint32_t& lo, uint32_t& hi, float v0, float v1, uint32_t h) {
  typedef float float2v __attribute__((ext_vector_type(2)));
  const float2v xv = {sr_hw_input(v0), sr_hw_input(v1)};
  const double x = __builtin_bit_cast(double, xv);  // the pair as one 64-bit register pair
  const uint32_t nh = ~h;  // 65535 - r16 in each half: r16(v0) = h & 0xFFFF, r16(v1) = h >> 16
  cvt_sr_pk<sel, sel == 0>(lo, x, (nh << 16) | 0xFFFFu);
  cvt_sr_pk<sel, sel == 0>(hi, x, (nh >> 1) | 0x7FFFu);
}

// Eight scaled values to eight SR codes, element 0 in the low nibble; h[p] is
// the hash of pair p (r16 of element 2p in its low half, 2p + 1 in its high).
__device__ __forceinline__ uint32_t sr_pack8(const float* v, const uint32_t* h) {
  uint32_t lo, hi;
  sr_pk<0>(lo, hi, v[0], v[1], h[0]);
  sr_pk<1>(lo, hi, v[2], v[3], h[1]);
  sr_pk<2>(lo, hi, v[4], v[5], h[2]);
  sr_pk<3>(lo, hi, v[6], v[7], h[3]);
  return (lo & 0x0F0F0F0Fu) | (hi & 0xF0F0F0F0u);
}

// Random bits of the SR hash: key = pcg(lo32(seed) ^ pcg(hi32(seed))); one
// pcg(key ^ (i >> 1)) per element pair, low half-word for the even element.
__host__ __forceinline__ uint32_t sr_key(uint64_t seed) {
  return pcg_host((uint32_t)seed ^ pcg_host((uint32_t)(seed >> 32)));
}

// Integer max over |bf16| pairs in a 32-bit word (sign bits cleared).
__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t acc, uint32_t w) {
  uint32_t a = w & 0x7FFF7FFFu;
  uint32_t lo = a & 0xFFFFu, hi = a >> 16;
  uint32_t m = lo > hi ? lo : hi;
  return acc > m ? acc : m;
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// FP32 -> BF16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Non-temporal stores of 16, 8, 4 and 1 bytes.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void st_nt(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}
__device__ __forceinline__ void st_nt(void* p, uint2 v) {
  __builtin_nontemporal_store(u32x2_t{v.x, v.y}, reinterpret_cast<u32x2_t*>(p));
}
__device__ __forceinline__ void st_nt(void* p, uint32_t v) {
  __builtin_nontemporal_store(v, reinterpret_cast<uint32_t*>(p));
}
__device__ __forceinline__ void st_nt8(uint8_t* p, uint8_t v) { __builtin_nontemporal_store(v, p); }

// One output element of a GEMM or a dequantization: FP32 as is, BF16 rounded
// to nearest even; load() reads one back as FP32.
template <typename OutT>
struct OutElem;
template <>
struct OutElem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float load_nt(const float* p) { return __builtin_nontemporal_load(p); }
  static __device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }
};
template <>
struct OutElem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p) { return __uint_as_float((uint32_t)*p << 16); }
  static __device__ __forceinline__ float load_nt(const uint16_t* p) {
    return __uint_as_float((uint32_t)__builtin_nontemporal_load(p) << 16);
  }
  static __device__ __forceinline__ void store_nt(uint16_t* p, float v) {
    __builtin_nontemporal_store((uint16_t)bf16_rne(v), p);
  }
};

// The random Hadamard transform y = (1/4) H16 diag(d) x (Sylvester H16,
// d_j = -1 where bit j of the sign mask is set) runs in three parts: the
// sign flips, applied by the loaders as they convert each element (sign_bit
// below), the radix-2 butterflies (fwht16), and the 1/4 normalization.

// 0x80000000 where bit j of the sign mask is set, else 0 (wave-uniform).
__device__ __forceinline__ uint32_t sign_bit(uint32_t sign_mask, int j) {
  return ((sign_mask >> j) & 1u) << 31;
}

// bf16 halves of a word as FP32 with the sign bit flipped by s (0 or
// 0x80000000): adding s to the top bit flips it (the carry drops out), so
// the low half costs one shift-add and the high half one and-xor.
__device__ __forceinline__ float bf16lo_signed(uint32_t w, uint32_t s) { return __uint_as_float((w << 16) + s); }
__device__ __forceinline__ float bf16hi_signed(uint32_t w, uint32_t s) {
  return __uint_as_float((w & 0xFFFF0000u) ^ s);
}
__device__ __forceinline__ float f32_signed(float x, uint32_t s) { return __uint_as_float(__float_as_uint(x) ^ s); }

// Radix-2 Walsh-Hadamard butterflies over 16 values, stages h = 1, 2, 4, 8,
// each pair (p, p + h) with (p & h) == 0 becoming (u_p + u_{p+h},
// u_p - u_{p+h}): u <- H16 u.
__device__ __forceinline__ void fwht16(float* u) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
    for (int p = 0; p < 16; p++) {
      if ((p & h) == 0) {
        float a = u[p], b = u[p + h];
        u[p] = a + b;
        u[p + h] = a - b;
      }
    }
  }
}

// Butterflies and the 1/4 normalization of already sign-flipped values.
__device__ __forceinline__ void rht16_signed(float* u) {
  fwht16(u);
#pragma unroll
  for (int j = 0; j < 16; j++) u[j] = 0.25f * u[j];
}

}  // namespace nvfp4
