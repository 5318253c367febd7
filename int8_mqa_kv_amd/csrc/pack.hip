// kv_pack_int8 kernel: quantise new tokens' K and V rows to symmetric int8
// with one fp32 scale per row and scatter them into their page records.
//
// The cache is int8 ("Character.AI: inference optimization", section 05) and
// K/V of a new token are computed once and kept ("Como funciona a inferência
// de IA", section "Por que o cache KV existe").  The coding of a row
// (wave_absmax, quant_scale, quant_code in device.hpp) is shared with the
// fused decode step, which codes the current token the same way, so both
// write the same bytes.
#include "internal.hpp"

namespace mqa {

constexpr int kPackWaves = 4;

template <int D, bool BF16>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (BF16) {
    return bf16_to_f32(static_cast<const uint16_t*>(base)[idx]);
  } else {
    return static_cast<const float*>(base)[idx];
  }
}

template <int D, bool BF16>
__global__ __launch_bounds__(kPackWaves * 64) void pack_kernel(
    const void* __restrict__ k, const void* __restrict__ v, int64_t num_tokens,
    int64_t row_stride, const int64_t* __restrict__ slot_mapping,
    uint8_t* __restrict__ pool, int64_t num_pages) {
  constexpr int PER = D / 64;  // channels per lane
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * kPackWaves + (threadIdx.x >> 6);
  if (t >= num_tokens) return;
  const int64_t slot = slot_mapping[t];
  if (slot < 0) return;
  const int64_t page = slot >> 4;
  const int j = (int)(slot & 15);
  if (page >= num_pages) return;
  uint8_t* rec = pool + page * (int64_t)page_bytes(D);

#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const void* src = which == 0 ? k : v;
    float x[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) x[e] = load_elem<D, BF16>(src, t * row_stride + lane * PER + e);
    const float a = wave_absmax<PER>(x);
    const float s = quant_scale(a);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int c = lane * PER + e;
      const int off = which == 0 ? k_code_offset(D, j, c) : v_code_offset(D, j, c);
      const int code = quant_code(x[e], a, s);
      rec[off] = code_byte(code);
    }
    if (lane == 0) {
      const int off = which == 0 ? k_scale_offset(D, j) : v_scale_offset(D, j);
      *reinterpret_cast<float*>(rec + off) = s;
    }
  }
}

hipError_t launch_pack(int D, bool bf16, const void* k, const void* v, int64_t num_tokens,
                       int64_t row_stride, const int64_t* slot_mapping, uint8_t* pool,
                       int64_t num_pages, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)((num_tokens + kPackWaves - 1) / kPackWaves));
  const dim3 block(kPackWaves * 64);
#define MQA_PACK(DD, BB)                                                                \
  hipLaunchKernelGGL((pack_kernel<DD, BB>), grid, block, 0, stream, k, v, num_tokens, \
                     row_stride, slot_mapping, pool, num_pages)
  if (D == 128) {
    if (bf16) MQA_PACK(128, true); else MQA_PACK(128, false);
  } else {
    if (bf16) MQA_PACK(64, true); else MQA_PACK(64, false);
  }
#undef MQA_PACK
  return hipGetLastError();
}

}  // namespace mqa
