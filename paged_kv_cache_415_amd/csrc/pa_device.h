// Device helpers shared by the gfx950 kernels: vector types, element
// conversions, the OCP E4M3FN encoder and wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- loads

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ uint32_t ld4(const void* p) { return *reinterpret_cast<const uint32_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Streaming loads (non-temporal hint): data read once, kept out of the way
// of the caches' normal replacement.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld8_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ uint32_t ld4_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// ------------------------------------------------------- 16-bit packing

// Two float32 -> packed 16-bit pair (round to nearest even), low half = a.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b);

template <>
__device__ __forceinline__ uint32_t pack2<__bf16>(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32 (RNE)
  return __builtin_bit_cast(uint32_t, v);
}

template <>
__device__ __forceinline__ uint32_t pack2<_Float16>(float a, float b) {
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  f16x2 v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
__device__ __forceinline__ float to_f32(T x) { return (float)x; }

// Low / high 16-bit halves of a dword as float.
template <typename T>
__device__ __forceinline__ float lo_f32(uint32_t w) {
  return (float)__builtin_bit_cast(T, (uint16_t)(w & 0xFFFFu));
}
template <typename T>
__device__ __forceinline__ float hi_f32(uint32_t w) {
  return (float)__builtin_bit_cast(T, (uint16_t)(w >> 16));
}

// ----------------------------------------------------- fp8 E4M3 decoding

// Two E4M3FN codes (bytes 0,1 of `w` when hi == false, bytes 2,3 when true)
// -> packed pair of 16-bit values of type T, exactly (every E4M3 value is
// representable in bf16 and in f16).  Uses gfx950's scaled conversion with
// scale 1.0.
template <typename T>
__device__ __forceinline__ uint32_t fp8x2_to(uint32_t w, bool hi);

template <>
__device__ __forceinline__ uint32_t fp8x2_to<__bf16>(uint32_t w, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
}

template <>
__device__ __forceinline__ uint32_t fp8x2_to<_Float16>(uint32_t w, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false));
}

// ----------------------------------------------------- int8 codes

// Two int8 codes (bytes 0,1 of `w` when hi == false, bytes 2,3 when true)
// -> packed pair of 16-bit values of type T, exactly (|code| <= 127 fits the
// 8 significant bits of bf16).
template <typename T>
__device__ __forceinline__ uint32_t i8x2_to(uint32_t w, bool hi) {
  const int s = hi ? 16 : 0;
  return pack2<T>((float)(int)(int8_t)(w >> s), (float)(int)(int8_t)(w >> (s + 8)));
}

// float32 -> symmetric int8 code under a positive scale: round half to even
// of one correctly rounded float32 division, clamped to [-127, 127]; NaN -> 0.
__device__ __forceinline__ int i8_encode(float x, float scale) {
  const float q = __builtin_rintf(x / scale);
  return q != q ? 0 : (int)fminf(fmaxf(q, -127.f), 127.f);
}

// ----------------------------------------------------- fp8 E4M3 encoding

// float32 -> OCP E4M3FN code, written from the format definition (1 sign,
// 4 exponent bits with bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, no
// infinities, 0x7F/0xFF NaN).  Round to nearest, ties to even; finite
// magnitudes above 448 and infinities saturate to 448; NaN -> 0x7F | sign.
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return sign | 0x7Fu;          // NaN
  if (mag >= 0x43E00000u) return sign | 0x7Eu;         // >= 448 (and inf): saturate
  if (mag < 0x3C800000u) {                             // below 2^-6: subnormal range
    // value = k * 2^-9 with k = round-half-even(|x| * 512); k == 8 is 2^-6,
    // whose code 0x08 continues the sequence.
    const float k = __builtin_rintf(__uint_as_float(mag) * 512.0f);
    return sign | (uint32_t)k;
  }
  // normal: exponent e in [-6, 8], keep 3 of the 23 mantissa bits, RNE
  const uint32_t e = (mag >> 23) - 127u + 7u;          // biased E4M3 exponent, 1..15
  const uint32_t m23 = mag & 0x7FFFFFu;
  uint32_t m3 = m23 >> 20;
  const uint32_t rest = m23 & 0xFFFFFu;
  if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) m3 += 1u;  // may carry into e
  uint32_t code = (e << 3) + m3;
  if (code > 0x7Eu) code = 0x7Eu;  // cannot happen below 448, kept as a guard
  return sign | code;
}

// Product rounded on its own (never fused into a following add): a logit
// formed this way minus the running max is exactly 0 for the max itself.
__device__ __forceinline__ float mul_rn(float a, float b) {
#pragma clang fp contract(off)
  return a * b;
}

// ------------------------------------------------- wave-level LDS order

// Order LDS accesses of different lanes of one wave (a wave's LDS
// instructions execute in order, so these cost no instruction): release
// after stores that other lanes of the wave will read, acquire before those
// reads, and before overwriting data that other lanes read.
__device__ __forceinline__ void wave_lds_release() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}
__device__ __forceinline__ void wave_lds_acquire() {
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ------------------------------------------------------ wave reductions

__device__ __forceinline__ float xor_max(float v, int mask) { return fmaxf(v, __shfl_xor(v, mask, 64)); }
__device__ __forceinline__ float xor_sum(float v, int mask) { return v + __shfl_xor(v, mask, 64); }

// Maximum that propagates NaN (v_maximum / v_maximum3_f32): unlike fmaxf it
// needs no canonicalisation of operands that come from lane moves.
__device__ __forceinline__ float fmax_nan(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48, with gfx950's
// row-swapping lane permutes: vector-ALU operations that, unlike the LDS
// path of __shfl_xor, add nothing to the LDS / scalar-memory counter, so a
// wait for them never waits for scalar loads in flight.
__device__ __forceinline__ float lanes4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmax_nan(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmax_nan(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Sum over the four lanes c16, c16 + 16, c16 + 32, c16 + 48 (every one of
// them gets the same total: each addition is commutative).
__device__ __forceinline__ float lanes4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Two 1.0 values of a 16-bit type, packed: the all-ones matrix operand whose
// product with a probability operand sums it.
template <typename T> inline constexpr uint32_t kOnes = 0;
template <> inline constexpr uint32_t kOnes<__bf16> = 0x3F803F80u;
template <> inline constexpr uint32_t kOnes<_Float16> = 0x3C003C00u;

// Byte permute: result byte k = sel byte k picks from {lo bytes 0-3 (0..3),
// hi bytes 0-3 (4..7)}; 0x0C gives a zero byte.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

}  // namespace pa
