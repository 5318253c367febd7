// Device helpers shared by the gfx950 kernels: vector types, exact int8 ->
// fp16 conversion, matrix-core wrapper, wavefront reductions.
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

// Four stored V bytes (one dword, byte k = code k + 128) -> four exact fp16
// values c + kVBias.  Each byte goes under the fp16 exponent of 1024 (bits
// 0x64uu = 1024 + u, exact for u < 1024) with one byte permute per pair, so
// the value is 1024 + 128 + c = 1152 + c.  A product of these with P carries
// kVBias * sum(P), which the caller removes once, from the same P summed on
// the matrix cores.
constexpr float kVBias = 1152.0f;
__device__ __forceinline__ void v_bytes_to_f16x4_biased(uint32_t u, f16x2& lo, f16x2& hi) {
  // v_perm_b32: selector bytes 0-3 pick bytes of the second operand, 4-7 of
  // the first.  Result bytes (low to high): u.b0, 0x64, u.b1, 0x64.
  lo = bitcast<f16x2>(__builtin_amdgcn_perm(0x64646464u, u, 0x04010400u));
  hi = bitcast<f16x2>(__builtin_amdgcn_perm(0x64646464u, u, 0x04030402u));
}

// D = A.B + C on one 16x16x32 fp16 tile, fp32 accumulate.  Lane l
// (i = l % 16, g = l / 16) supplies A[i][8g..8g+7] and B[8g..8g+7][i] and
// receives D[4g..4g+3][i].
__device__ __forceinline__ f32x4 mma16(const f16x8& a, const f16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D = A.B + C on one 16x16x64 int8 tile, int32 accumulate (exact).  Lane l
// (i = l % 16, g = l / 16) supplies A[i][16g..16g+15] and B[16g..16g+15][i]
// (16 bytes each) and receives D[4g..4g+3][i].
__device__ __forceinline__ i32x4 mma_i8(const u32x4& a, const u32x4& b, const i32x4& c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(bitcast<i32x4>(a), bitcast<i32x4>(b), c, 0, 0, 0);
}

// A query element as a 15-bit fixed-point integer v = rint(x * sc)
// (|x * sc| < 2^14) split into two int8 halves v = 256*hi + lo with
// hi = floor((v + 128) / 256) in [-64, 64] and lo = v - 256*hi in [-128, 127].
// fma(x, sc, 1.5*2^23 + 128) lands on the fp32 grid of spacing 1 (the FMA
// rounds half to even, as rint does), so the low 16 bits of its bits hold
// t = v + 128 in two's complement: byte 1 of t is hi, byte 0 xor 0x80 is lo.
__device__ __forceinline__ uint32_t q15_word(float x, float sc) {
  return bitcast<uint32_t>(__builtin_fmaf(x, sc, 12583040.0f));  // 1.5*2^23 + 128
}
// hi and lo int8 halves of four q15_words, packed (element k = byte k)
__device__ __forceinline__ void q15_pack4(uint32_t t0, uint32_t t1, uint32_t t2, uint32_t t3,
                                          uint32_t& hi, uint32_t& lo) {
  // v_perm_b32 selector bytes 0-3 pick the second operand's bytes, 4-7 the first's
  const uint32_t a = __builtin_amdgcn_perm(t1, t0, 0x05010400u);  // t0.b0 t1.b0 t0.b1 t1.b1
  const uint32_t b = __builtin_amdgcn_perm(t3, t2, 0x05010400u);  // t2.b0 t3.b0 t2.b1 t3.b1
  lo = __builtin_amdgcn_perm(b, a, 0x05040100u) ^ 0x80808080u;
  hi = __builtin_amdgcn_perm(b, a, 0x07060302u);
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
