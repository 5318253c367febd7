// A streaming read of device memory: how fast can this GPU move bytes from
// HBM into its compute units?  Decode attention over the int8 cache is a
// stream of KV bytes ("Character.AI: inference optimization", section 02:
// the KV cache's size sets the I/O cost of attention), so the bandwidth a
// plain read reaches on the machine is the yardstick its kernels are held
// to, beside the published peak.  Not part of the method.
//
// Every workgroup XORs a contiguous range of 16-byte words (eight 128-bit
// loads in flight per lane) and writes one 32-bit word, so the result -- the
// XOR of every 32-bit word of the buffer, after folding the workgroups'
// words -- is checkable and the loads cannot be dropped.
#include "internal.hpp"

namespace mqa {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_kernel(const u32x4* __restrict__ src,
                                                                 int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  const int64_t per_wg = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per_wg;
  const int64_t end = min(beg + per_wg, n16);
  uint32_t acc = 0;
  int64_t i = beg + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * kProbeThreads < end; i += kProbeUnroll * kProbeThreads) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = src[i + u * kProbeThreads];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < end; i += kProbeThreads) {
    const u32x4 v = src[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t part[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) x ^= part[w];
    sink[blockIdx.x] = x;
  }
}

hipError_t launch_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int groups,
                           hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3((unsigned)groups), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace mqa
