// Internal device helpers shared by the cpattn HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cpattn.h"

namespace cpattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Two fp32 -> packed bf16 pair, round to nearest even (gfx950 has a native
// instruction for this conversion).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x[lane], x[lane ^ 32]) in every lane: v_permlane32_swap exchanges the two
// 32-lane halves of a wave register to register, without a round trip through LDS.
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max(x[lane], x[lane ^ 16]) in every lane: v_permlane16_swap exchanges the
// odd and even 16-lane rows of a wave register to register.
__device__ __forceinline__ float max_across_rows16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Element loads of an input row: 8 consecutive elements widened to fp32.
template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static __device__ __forceinline__ void load8(const float *p, float (&o)[8]) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t *>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t *>(p + 4);
    o[0] = a[0]; o[1] = a[1]; o[2] = a[2]; o[3] = a[3];
    o[4] = b[0]; o[5] = b[1]; o[6] = b[2]; o[7] = b[3];
  }
  static __device__ __forceinline__ float load1(const float *p) { return *p; }
};

template <>
struct Elem<__bf16> {
  static __device__ __forceinline__ void load8(const __bf16 *p, float (&o)[8]) {
    const u32x4_t w = *reinterpret_cast<const u32x4_t *>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ float load1(const __bf16 *p) {
    return bf16_bits_to_f32(*reinterpret_cast<const uint16_t *>(p));
  }
};

// Merge of an online-softmax triple (m1, d1) with (m2, d2): returns the
// weights a1 = exp(m1 - m), a2 = exp(m2 - m) for m = max(m1, m2), with a weight
// of 0 for a side whose max is -inf (the identity).
__device__ __forceinline__ void merge_weights(float m1, float m2, float &m, float &a1, float &a2) {
  m = fmaxf(m1, m2);
  a1 = (m1 == kNegInf) ? 0.f : expf(m1 - m);
  a2 = (m2 == kNegInf) ? 0.f : expf(m2 - m);
}

// Validation of a prefill description and (rank, step) shared by the ring-step
// entry points (CPATTN_OK or the error code; no device call).
__attribute__((visibility("hidden"))) int check_prefill(const cpattn_prefill_desc *desc, int32_t rank,
                                                          int32_t step);
// CPATTN_OK when every sequence of a description check_prefill accepted fits
// the ring-step launches (the error cpattn_ring_step_partial would return
// otherwise, before launching anything).
__attribute__((visibility("hidden"))) int check_launches(const cpattn_prefill_desc *desc);
// Rows of one rank's local buffers (sum over sequences of 2 c_i, pad rows
// included) for a description check_prefill accepted.
__attribute__((visibility("hidden"))) int64_t local_rows(const cpattn_prefill_desc *desc);

}  // namespace cpattn
