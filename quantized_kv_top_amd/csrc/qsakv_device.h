// Device-side helpers shared by the qsakv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qsakv {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

template <typename T>
__device__ __forceinline__ T bitcast(const auto& x) { return __builtin_bit_cast(T, x); }

// ---------------------------------------------------------------------------
// wave reductions (shuffle based; used outside the hot loop or on few values)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
// Reduce across the four 16-lane groups that share lane & 15.  gfx950's
// permlane swaps exchange 32-lane halves and odd/even 16-lane rows in the
// VALU (no LDS round trip): called with the same value as both operands,
// the pair returned holds x[l] and x[l ^ 32] (then x[l ^ 16]) in some order.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float group4_max(float x) { return xor32_max(xor16_max(x)); }
// the two pairings are summed in the same order on every lane, so all four
// groups end with bitwise the same total
__device__ __forceinline__ float group4_sum(float x) { return xor32_sum(xor16_sum(x)); }

// ---------------------------------------------------------------------------
// exact conversions of cache codes to MFMA operands
// ---------------------------------------------------------------------------
// Byte permute: result byte k = byte sel.k of the 8-byte value {hi, lo}
// (selector 0..3 -> lo bytes, 4..7 -> hi bytes).
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two signed int8 codes in bytes (b_lo, b_hi) of `x` -- already XOR-ed with
// 0x80 so that each byte holds q + 128 -- become the fp16 pair
// (1152 + q_lo, 1152 + q_hi): 0x64XX is the fp16 value 1024 + XX, exact for
// XX < 256.  The constant 1152 is taken off before the MFMA (i8pair_unbias).
__device__ __forceinline__ uint32_t i8pair_to_f16x2(uint32_t x_biased, uint32_t sel) {
  return perm(0x64646464u, x_biased, sel);
}
constexpr uint32_t kSelB01 = 0x04010400u;  // bytes 0,1 -> (0x64b0, 0x64b1)
constexpr uint32_t kSelB23 = 0x04030402u;  // bytes 2,3 -> (0x64b2, 0x64b3)
// (1152 + q_lo, 1152 + q_hi) -> (q_lo, q_hi): one packed fp16 subtract,
// exact (both operands and the difference are integers below 2^11).
__device__ __forceinline__ uint32_t i8pair_unbias(uint32_t h) {
  const f16x2 b = {(_Float16)1152.f, (_Float16)1152.f};
  return bitcast<uint32_t>(bitcast<f16x2>(h) - b);
}

// Two OCP E4M3FN codes in the low (hi_word = false) or high 16 bits of w ->
// two exact fp16 values (every E4M3 value is representable in fp16), using
// gfx950's OCP-FP8 conversion with unit scale.
template <bool kHiWord>
__device__ __forceinline__ uint32_t e4m3pair_to_f16x2(uint32_t w) {
  f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHiWord);
  return bitcast<uint32_t>(h);
}
// The two FP4 E2M1 codes in byte kByte of w -> the fp16 pair (low nibble,
// high nibble): gfx950's FP4 conversion with unit scale (exact: every E2M1
// value is an fp16 value).
template <int kByte>
__device__ __forceinline__ uint32_t e2m1pair_to_f16x2(uint32_t w) {
  f16x2 h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, kByte);
  return bitcast<uint32_t>(h);
}
// ---------------------------------------------------------------------------
// MFMA 16x16x32 (fp16 / bf16 inputs, fp32 accumulate)
//   A (16 x 32): lane l holds row l%16, k-slots 8*(l/16) .. +7
//   B (32 x 16): lane l holds col l%16, the same k-slots
//   C (16 x 16): lane l holds rows 4*(l/16) .. +3 of col l%16
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace qsakv
