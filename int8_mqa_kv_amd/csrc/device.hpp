// Device helpers shared by the gfx950 kernels: vector types, exact int8 ->
// fp16 conversion, two-term fp16 splits, matrix-core wrapper, wavefront
// reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.hpp"

namespace mqa {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T, typename F>
__device__ __forceinline__ T bitcast(F f) {
  static_assert(sizeof(T) == sizeof(F), "size");
  return __builtin_bit_cast(T, f);
}

// Four stored code bytes (one dword, byte k = code k + 128: K and V codes
// are both stored with the sign bit flipped) -> four exact fp16 values
// c + kCodeBias.  Each byte goes under the fp16 exponent of 1024 (bits
// 0x64uu = 1024 + u, exact for u < 1024) with one byte permute per pair, so
// the value is 1024 + 128 + c = 1152 + c.  A product of these with another
// operand carries kCodeBias times that operand's sum, which the caller
// removes: for Q.K^T through the accumulator's starting value, for P.V from
// a product of the same P with an all-ones operand.
constexpr float kCodeBias = 1152.0f;
__device__ __forceinline__ void codes_to_f16x4_biased(uint32_t u, f16x2& lo, f16x2& hi) {
  // v_perm_b32: selector bytes 0-3 pick bytes of the second operand, 4-7 of
  // the first.  Result bytes (low to high): u.b0, 0x64, u.b1, 0x64.
  lo = bitcast<f16x2>(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
  hi = bitcast<f16x2>(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
}
// Eight stored code bytes (two dwords) -> one fp16 matrix-core operand.
__device__ __forceinline__ f16x8 codes_to_f16x8_biased(uint32_t w0, uint32_t w1) {
  f16x2 a0, a1, b0, b1;
  codes_to_f16x4_biased(w0, a0, a1);
  codes_to_f16x4_biased(w1, b0, b1);
  return f16x8{a0[0], a0[1], a1[0], a1[1], b0[0], b0[1], b1[0], b1[1]};
}

// D = A.B + C on one 16x16x32 fp16 tile, fp32 accumulate.  Lane l
// (i = l % 16, g = l / 16) supplies A[i][8g..8g+7] and B[8g..8g+7][i] and
// receives D[4g..4g+3][i].
__device__ __forceinline__ f32x4 mma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// fp16(x - h) for an fp32 value x and an fp16 value h held in the low
// (HI = false) or high (HI = true) half of a packed register, written into the
// same half of d by one mixed-precision FMA (the rest is formed exactly and
// rounded to fp16 once).  The low-half form leaves d's high half as it was,
// the high-half form its low half.
__device__ __forceinline__ void sub_f16_lo(uint32_t& d, float x, f16x2 h) {
  asm("v_fma_mixlo_f16 %0, -%1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(x));
}
__device__ __forceinline__ void sub_f16_hi(uint32_t& d, float x, f16x2 h) {
  asm("v_fma_mixhi_f16 %0, -%1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(d) : "v"(h), "v"(x));
}

// Two fp32 values as a two-term fp16 pair each: hi = fp16(x) and
// lo = fp16(x - hi).  |x - hi| <= 2^-11 |x| and lo rounds that rest once
// more, so |hi + lo - x| <= 2^-22 |x| + 2^-25 (the last term: a rest below
// fp16's normal range is kept to fp16's subnormal spacing).
__device__ __forceinline__ void split_f16x2(float x0, float x1, f16x2& hi, f16x2& lo) {
  hi = f16x2{(_Float16)x0, (_Float16)x1};
  uint32_t r;
  sub_f16_lo(r, x0, hi);
  sub_f16_hi(r, x1, hi);
  lo = bitcast<f16x2>(r);
}

// Reductions across the four lanes i, i+16, i+32, i+48 (one matrix row) with
// the gfx950 lane swaps: permlane16_swap(x, x) returns {x[l], x[l^16]} in some
// order on every lane (permlane32_swap likewise for l^32), so one swap and one
// max or add combine a lane with its partner without going through LDS.
// The larger of two floats as one v_max_f32.  fmaxf on values fresh from a
// lane swap first quiets each operand with a v_max_f32 of its own (IEEE mode
// requires it for signalling NaNs, and no operand here is one).
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false,
                                                  false);
  return max2(bitcast<float>((uint32_t)r[0]), bitcast<float>((uint32_t)r[1]));
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false,
                                                  false);
  return max2(bitcast<float>((uint32_t)r[0]), bitcast<float>((uint32_t)r[1]));
}
__device__ __forceinline__ float xor16_add(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false,
                                                  false);
  return bitcast<float>((uint32_t)r[0]) + bitcast<float>((uint32_t)r[1]);
}
__device__ __forceinline__ float xor32_add(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(bitcast<uint32_t>(x), bitcast<uint32_t>(x), false,
                                                  false);
  return bitcast<float>((uint32_t)r[0]) + bitcast<float>((uint32_t)r[1]);
}
__device__ __forceinline__ float row_max4(float x) { return xor32_max(xor16_max(x)); }
__device__ __forceinline__ float row_sum4(float x) { return xor32_add(xor16_add(x)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Exponent E of x = m * 2^E with m in [0.5, 1) (x > 0, subnormals handled).
__device__ __forceinline__ int frexp_exp(float x) { return __builtin_amdgcn_frexp_expf(x); }
__device__ __forceinline__ float ldexp2(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return bitcast<float>((uint32_t)b << 16);
}

// ---------------------------------------------------------------------------
// Symmetric int8 coding of one K or V row with one fp32 scale
// ("Character.AI: inference optimization", section 05: the KV cache is int8):
//   a = max|x|,  s = a / 127 (fp32),  code = clamp(rint(x / s), -127, 127)
// with IEEE fp32 division (hipcc's default `/` is correctly rounded) and
// round-half-to-even; a = 0 gives s = 0 and zero codes.
// ---------------------------------------------------------------------------
// max |x| over a wavefront's PER values per lane; every lane gets the result
template <int PER>
__device__ __forceinline__ float wave_absmax(const float (&x)[PER]) {
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < PER; ++e) a = fmaxf(a, fabsf(x[e]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  return a;
}
__device__ __forceinline__ float quant_scale(float a) { return a / 127.0f; }
__device__ __forceinline__ int quant_code(float x, float a, float s) {
  if (a == 0.0f) return 0;
  const float r = __builtin_rintf(x / s);
  return (int)fminf(fmaxf(r, -127.0f), 127.0f);
}

}  // namespace mqa
