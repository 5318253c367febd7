// Grouped-query bf16 decode: the baseline the multi-query int8 cache is
// measured against.
//
// "Character.AI: inference optimization", section 03, technique table: the
// multi-query design cuts the KV cache 8X against grouped-query attention.
// To show that in bytes and in time on the same harness, this file holds a
// plain GQA decode path: num_kv_heads K/V heads per layer in bf16, each
// shared by num_q_heads / num_kv_heads query heads, paged in 16-token pages.
//
// Page record (one per 16 tokens, all KV heads): for KV head h, 64*d bytes at
// h*64*d, holding that head's 16 tokens as K (32*d bytes) then V (32*d bytes),
// bf16, each in bf16 matrix-core operand order so that a lane reads its 16
// (K) or 8 (V) bytes at a fixed place:
//   K, channel c of token j:  (c/32)*1024 + (16*((c%32)/8) + j)*16 + (c%8)*2
//   V, channel c of token j:  32*d + (c/16)*512 + (16*(j/4) + c%16)*8 + (j%4)*2
// QK^T runs on bf16 matrix cores with q in bf16 (exact products); P is split
// into two bf16 halves (hi, and the rounding rest) so that PV keeps about 16
// bits of P with V as stored.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/mqa_kv.h"
#include "internal.hpp"

namespace mqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGqaWaves = 8;          // wavefronts per decode workgroup
constexpr int kGqaMaxGroup = 16;      // query heads per KV head, at most (one 16-row tile)

MQA_HD constexpr int gqa_head_page_bytes(int D) { return 64 * D; }

struct GqaArgs {
  int64_t num_pages;
  int32_t max_pages, max_context, batch, num_q_heads, num_kv_heads, group, window;
  int32_t nchunk, total_wgs;
  uint32_t ch_recip;
  float scale_log2;
};

__device__ __forceinline__ f32x4 mma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Pack: one wavefront per (token, KV head) writes its K and V rows into place.
template <int D>
__global__ __launch_bounds__(256) void gqa_pack_kernel(const uint16_t* __restrict__ k,
                                                       const uint16_t* __restrict__ v,
                                                       int64_t num_tokens, int32_t num_kv_heads,
                                                       const int64_t* __restrict__ slot_mapping,
                                                       uint8_t* __restrict__ pool,
                                                       int64_t num_pages) {
  const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= num_tokens * num_kv_heads) return;
  const int64_t t = item / num_kv_heads;
  const int h = (int)(item % num_kv_heads);
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || (slot >> 4) >= num_pages) return;
  const int j = (int)(slot & 15);
  uint8_t* rec = pool + (slot >> 4) * (int64_t)num_kv_heads * gqa_head_page_bytes(D) +
                 (int64_t)h * gqa_head_page_bytes(D);
  const int lane = threadIdx.x & 63;
  for (int c = lane; c < D; c += 64) {
    const uint16_t kc = k[(t * num_kv_heads + h) * D + c];
    const uint16_t vc = v[(t * num_kv_heads + h) * D + c];
    *reinterpret_cast<uint16_t*>(rec + (c / 32) * 1024 + (16 * ((c % 32) / 8) + j) * 16 + (c % 8) * 2) = kc;
    *reinterpret_cast<uint16_t*>(rec + 32 * D + (c / 16) * 512 + (16 * (j / 4) + c % 16) * 8 +
                                 (j % 4) * 2) = vc;
  }
}

// ---------------------------------------------------------------------------
// Decode: one workgroup = one (sequence, KV head, chunk of pages); each of its
// wavefronts streams its share of the pages through its own LDS slot (one
// block of two pages, refilled as soon as the block is in registers) and
// keeps an online softmax for the group's query rows; the wavefronts merge in
// LDS, then the workgroup writes the output or its chunk's partial record.
constexpr int kGqaVmcnt0 = 0x0F70;     // s_waitcnt: vmcnt(0)
constexpr int kGqaLgkm0 = 0xC07F;      // s_waitcnt: lgkmcnt(0)
constexpr float kGqaTau = 8.0f;        // lazy rescale threshold (log2 units)

template <int D>
struct alignas(16) GqaLds {
  uint8_t slot[kGqaWaves][2][gqa_head_page_bytes(D)];
  float m[kGqaWaves][16];
  float l[kGqaWaves][16];
};

template <int D>
__global__ __launch_bounds__(kGqaWaves * 64) void gqa_decode_kernel(
    const GqaArgs a, const uint16_t* __restrict__ q, float* __restrict__ out,
    const uint8_t* __restrict__ pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ context_lens, float* __restrict__ ws) {
  constexpr int W = kGqaWaves, KS = D / 32, VT = D / 16, HP = gqa_head_page_bytes(D);
  __shared__ GqaLds<D> sm;
  static_assert(sizeof(GqaLds<D>) <= 160 * 1024, "LDS");
  static_assert(VT * 64 * 16 <= HP, "accumulator dump fits a page slot");
  const int wg = blockIdx.x;
  if (wg >= a.total_wgs) return;
  const uint32_t item = __umulhi((uint32_t)wg, a.ch_recip);
  uint32_t it = item, chunk = (uint32_t)wg - it * (uint32_t)a.nchunk;
  if (chunk >= (uint32_t)a.nchunk) {  // one correction step of the reciprocal
    ++it;
    chunk -= (uint32_t)a.nchunk;
  }
  const int seq = (int)(it / (uint32_t)a.num_kv_heads);
  const int head = (int)(it % (uint32_t)a.num_kv_heads);
  const int G = a.group;
  const int lane = threadIdx.x & 63, li = lane & 15, lg = lane >> 4;
  const int wv = threadIdx.x >> 6;

  // query rows of the group as the B operand: lane (i, g), k-step s holds
  // row i, channels 32s + 8g .. +7 (rows past the group are zero)
  bf16x8 qop[KS];
  const int64_t qrow0 = (int64_t)seq * a.num_q_heads + (int64_t)head * G;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4 x = u32x4{0, 0, 0, 0};
    if (li < G) x = *reinterpret_cast<const u32x4*>(q + (qrow0 + li) * D + 32 * s + 8 * lg);
    qop[s] = __builtin_bit_cast(bf16x8, x);
  }
  const int cap = (int)min<int64_t>(a.max_context, (int64_t)a.max_pages * 16);
  const int ctx = min(max(context_lens[seq], 0), cap);
  const int hi = ctx, lo = a.window > 0 ? max(0, ctx - a.window) : 0;
  const int p_first = lo >> 4, p_last = hi > lo ? (hi - 1) >> 4 : p_first - 1;
  const int np = p_last - p_first + 1;
  const int nch = np > 0 ? min(a.nchunk, max(1, (np + 2 * W - 1) / (2 * W))) : 1;
  if ((int)chunk >= nch) return;
  const int cbeg = p_first + (int)((uint32_t)(chunk * max(np, 0)) / (uint32_t)nch);
  const int npc = p_first + (int)((uint32_t)((chunk + 1) * max(np, 0)) / (uint32_t)nch) - cbeg;
  const int pbeg = cbeg + wv * npc / W, pend = cbeg + (wv + 1) * npc / W;
  const int32_t* row = block_table + (int64_t)seq * a.max_pages;
  const int ids = pbeg + lane < pend ? row[pbeg + lane] : -1;
  auto page_ok = [&](int pi, int& pid) {
    pid = __builtin_amdgcn_readlane(ids, min(max(pi - pbeg, 0), 63));
    return pi < pend && (uint32_t)pid < (uint64_t)a.num_pages;
  };
  const int64_t head_off = (int64_t)head * HP;
  const int64_t page_stride = (int64_t)a.num_kv_heads * HP;
  auto issue = [&](int pa) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int pid;
      const bool ok = page_ok(pa + u, pid);
      const uint8_t* src = pool + (ok ? (int64_t)pid : 0) * page_stride + head_off + lane * 16;
      uint8_t* dst = &sm.slot[wv][u][0];
      // each workgroup reads only its KV head's part of a page, so nothing
      // reuses these bytes: non-temporal (the cache-policy operand's nt bit),
      // as the multi-query decode does for pages with one reader
#pragma unroll
      for (int piece = 0; piece < HP / 1024; ++piece)
        __builtin_amdgcn_global_load_lds(src + piece * 1024, dst + piece * 1024, 16, 0, 2);
    }
  };
  const int nblk = (pend - pbeg + 1) >> 1;
  if (nblk > 0) issue(pbeg);

  f32x4 acc[VT];
#pragma unroll
  for (int t = 0; t < VT; ++t) acc[t] = f32x4{0, 0, 0, 0};
  float m = -__builtin_inff(), l = 0.0f;
  const float c = a.scale_log2;
  for (int b = 0; b < nblk; ++b) {
    const int pa = pbeg + 2 * b;
    // the block's pages have landed (the only loads outstanding)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kGqaVmcnt0);
    __builtin_amdgcn_sched_barrier(0);
    u32x4 kr[2][KS];
    u32x2 vr[2][VT];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint8_t* sp = &sm.slot[wv][u][0];
#pragma unroll
      for (int s = 0; s < KS; ++s) kr[u][s] = *reinterpret_cast<const u32x4*>(sp + s * 1024 + lane * 16);
#pragma unroll
      for (int t = 0; t < VT; ++t)
        vr[u][t] = *reinterpret_cast<const u32x2*>(sp + 32 * D + t * 512 + lane * 8);
    }
    int pid0, pid1;
    const bool ok0 = page_ok(pa, pid0), ok1 = page_ok(pa + 1, pid1);
    // the slot is free once the reads above completed: the next block flies
    // while this one is computed
    __builtin_amdgcn_s_waitcnt(kGqaLgkm0);
    __builtin_amdgcn_sched_barrier(0);
    if (b + 1 < nblk) issue(pa + 2);

    f32x4 s2[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 sc = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int s = 0; s < KS; ++s) sc = mma_bf16(__builtin_bit_cast(bf16x8, kr[u][s]), qop[s], sc);
      s2[u] = sc;
    }
    // scores in log2 units; keys outside [lo, hi) or on a bad page are -inf
    float t8[8];
    float mb = -__builtin_inff();
    uint32_t vkeep[2][2];  // per page, per V dword (two keys): bits of the keys kept
    bool all_valid = true;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      bool valid[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pos = (pa + u) * 16 + 4 * lg + r;
        valid[r] = (u ? ok1 : ok0) && pos >= lo && pos < hi;
        all_valid &= valid[r];
        const float x = s2[u][r] * c;
        t8[4 * u + r] = valid[r] ? x : -__builtin_inff();
        mb = fmaxf(mb, t8[4 * u + r]);
      }
#pragma unroll
      for (int w = 0; w < 2; ++w)
        vkeep[u][w] = (valid[2 * w] ? 0x0000FFFFu : 0u) | (valid[2 * w + 1] ? 0xFFFF0000u : 0u);
    }
    // A masked key's V may be anything (a page past the context, bytes never
    // written, NaN): P = 0 does not cancel NaN in the product, so the key's V
    // elements are zeroed.  A lane's V operand covers exactly the keys of its
    // own P values, so its own mask applies.
    if (__builtin_amdgcn_ballot_w64(!all_valid) != 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int t = 0; t < VT; ++t) {
          vr[u][t][0] &= vkeep[u][0];
          vr[u][t][1] &= vkeep[u][1];
        }
    }
    mb = row_max4(mb);
    const bool move = mb > m + kGqaTau;
    const float m_new = move ? mb : m;
    const float alpha = move ? fast_exp2(m - m_new) : 1.0f;
    const float neg = m_new == -__builtin_inff() ? 0.0f : -m_new;
    float p8[8];
    float ps = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p8[e] = fast_exp2(t8[e] + neg);
      ps += p8[e];
    }
    l = l * alpha + ps;
    m = m_new;
    if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
      for (int t = 0; t < VT; ++t) acc[t] *= alpha;
    }
    // P^T operand as two bf16 halves: hi = bf16(p), lo = bf16(p - hi)
    bf16x8 ph, pl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      ph[e] = (__bf16)p8[e];
      pl[e] = (__bf16)(p8[e] - (float)ph[e]);
    }
#pragma unroll
    for (int t = 0; t < VT; ++t) {
      const u32x4 vw = u32x4{vr[0][t][0], vr[0][t][1], vr[1][t][0], vr[1][t][1]};
      const bf16x8 va = __builtin_bit_cast(bf16x8, vw);
      acc[t] = mma_bf16(va, ph, acc[t]);
      acc[t] = mma_bf16(va, pl, acc[t]);
    }
  }

  // ---- merge the W wavefronts in LDS ----
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kGqaVmcnt0);
  const float lrow = row_sum4(l);
  if (lg == 0) {
    sm.m[wv][li] = m;
    sm.l[wv][li] = lrow;
  }
  f32x4* dump = reinterpret_cast<f32x4*>(&sm.slot[wv][0][0]);
#pragma unroll
  for (int t = 0; t < VT; ++t) dump[t * 64 + lane] = acc[t];
  __syncthreads();
  for (int t = wv; t < VT; t += W) {
    float mm = -__builtin_inff();
#pragma unroll
    for (int x = 0; x < W; ++x) mm = fmaxf(mm, sm.m[x][li]);
    const float mu = mm == -__builtin_inff() ? 0.0f : mm;
    float ll = 0.0f;
    f32x4 o = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int x = 0; x < W; ++x) {
      const float e = fast_exp2(sm.m[x][li] - mu);
      ll += e * sm.l[x][li];
      o += e * reinterpret_cast<const f32x4*>(&sm.slot[x][0][0])[t * 64 + lane];
    }
    if (li >= G) continue;
    if (nch == 1) {
      const float inv = ll > 0.0f ? 1.0f / ll : 0.0f;
      *reinterpret_cast<f32x4*>(out + (qrow0 + li) * D + 16 * t + 4 * lg) = o * inv;
    } else {
      // partial record of (item, chunk): m[16], l[16], acc[16][D]
      float* rec = ws + ((int64_t)it * a.nchunk + chunk) * (32 + 16 * D);
      if (lg == 0 && t == wv) {
        rec[li] = mm;
        rec[16 + li] = ll;
      }
      *reinterpret_cast<f32x4*>(rec + 32 + li * D + 16 * t + 4 * lg) = o;
    }
  }
}

// Chunks of a split (sequence, KV head): one workgroup per item folds its
// chunks' records in chunk order and writes the group's rows.
template <int D>
__global__ __launch_bounds__(256) void gqa_merge_kernel(const GqaArgs a, float* __restrict__ out,
                                                        const int32_t* __restrict__ context_lens,
                                                        const float* __restrict__ ws) {
  const int it = blockIdx.x;
  const int seq = it / a.num_kv_heads, head = it % a.num_kv_heads;
  const int cap = (int)min<int64_t>(a.max_context, (int64_t)a.max_pages * 16);
  const int ctx = min(max(context_lens[seq], 0), cap);
  const int lo = a.window > 0 ? max(0, ctx - a.window) : 0;
  if (ctx <= lo) return;  // the decode kernel wrote zeros
  const int np = ((ctx - 1) >> 4) - (lo >> 4) + 1;
  const int nch = min(a.nchunk, max(1, (np + 2 * kGqaWaves - 1) / (2 * kGqaWaves)));
  if (nch == 1) return;  // written by the decode kernel
  const int64_t qrow0 = (int64_t)seq * a.num_q_heads + (int64_t)head * a.group;
  for (int e = threadIdx.x; e < a.group * D; e += blockDim.x) {
    const int r = e / D, d = e % D;
    float mm = -__builtin_inff();
    for (int k = 0; k < nch; ++k)
      mm = fmaxf(mm, ws[((int64_t)it * a.nchunk + k) * (32 + 16 * D) + r]);
    const float mu = mm == -__builtin_inff() ? 0.0f : mm;
    float ll = 0.0f, o = 0.0f;
    for (int k = 0; k < nch; ++k) {
      const float* rec = ws + ((int64_t)it * a.nchunk + k) * (32 + 16 * D);
      const float f = fast_exp2(rec[r] - mu);
      ll += f * rec[16 + r];
      o += f * rec[32 + r * D + d];
    }
    out[(qrow0 + r) * D + d] = ll > 0.0f ? o / ll : 0.0f;
  }
}

}  // namespace mqa

using namespace mqa;

namespace {

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255) == 0; }

int gqa_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t max_context,
             int32_t window, int32_t head_dim, GqaArgs& a, size_t& ws_bytes) {
  if (batch < 0 || num_kv_heads < 1 || num_q_heads < 1 || num_q_heads % num_kv_heads)
    return fail(MQA_ERR_INVALID, "heads: %d query heads over %d KV heads", num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > kGqaMaxGroup)
    return fail(MQA_ERR_UNSUPPORTED, "more than %d query heads per KV head", kGqaMaxGroup);
  if (head_dim != 64 && head_dim != 128) return fail(MQA_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (max_context < 0 || window < 0) return fail(MQA_ERR_INVALID, "negative context or window");
  // (bounded so that the kernel's 32-bit chunk boundaries cannot wrap)
  if (max_context > MQA_MAX_CONTEXT)
    return fail(MQA_ERR_UNSUPPORTED, "max_context %d above %d", max_context, MQA_MAX_CONTEXT);
  const int64_t ctx_pages = (max_context + 15) / 16;
  const int64_t max_np = window > 0 ? std::min<int64_t>((window + 15) / 16 + 1, ctx_pages) : ctx_pages;
  const int64_t items = (int64_t)batch * num_kv_heads;
  const int64_t target = std::max<int64_t>(256, items);
  const int64_t need = (max_np + 64 * kGqaWaves - 1) / (64 * kGqaWaves);
  const int64_t nchunk = std::max<int64_t>({1, target / std::max<int64_t>(items, 1), need});
  // one dispatch holds at most 2^32 - 1 work-items
  if (items * nchunk * kGqaWaves * 64 > INT64_C(0xFFFFFFFF))
    return fail(MQA_ERR_UNSUPPORTED, "launch too large: %lld workgroups", (long long)(items * nchunk));
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.window = window;
  a.max_context = max_context;
  a.nchunk = (int)nchunk;
  a.total_wgs = (int)(items * nchunk);
  a.ch_recip = 0xFFFFFFFFu / (uint32_t)nchunk;
  ws_bytes = nchunk > 1 ? (size_t)(items * nchunk * (32 + 16 * head_dim)) * sizeof(float) : 0;
  return MQA_OK;
}

}  // namespace

extern "C" {

size_t mqa_gqa_page_bytes(int32_t num_kv_heads, int32_t head_dim) {
  if (num_kv_heads < 1 || (head_dim != 64 && head_dim != 128)) return 0;
  return (size_t)num_kv_heads * gqa_head_page_bytes(head_dim);
}

int mqa_gqa_pack_bf16(const void* k, const void* v, int64_t num_tokens, const int64_t* slot_mapping,
                      void* pool, int64_t num_pages, int32_t num_kv_heads, int32_t head_dim,
                      void* stream) {
  if (num_tokens < 0) return fail(MQA_ERR_INVALID, "num_tokens < 0");
  if (num_kv_heads < 1) return fail(MQA_ERR_INVALID, "num_kv_heads < 1");
  if (head_dim != 64 && head_dim != 128) return fail(MQA_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (num_tokens * num_kv_heads > MQA_PACK_MAX_TOKENS)
    return fail(MQA_ERR_UNSUPPORTED, "%lld (token, KV head) pairs above %d per call",
                (long long)num_tokens * num_kv_heads, MQA_PACK_MAX_TOKENS);
  if (num_tokens == 0) return ok();
  if (!k || !v || !slot_mapping || !pool) return fail(MQA_ERR_INVALID, "NULL pointer");
  if (num_pages <= 0 || !aligned256(pool)) return fail(MQA_ERR_INVALID, "bad pool");
  const int64_t items = num_tokens * num_kv_heads;
  const dim3 grid((unsigned)((items + 3) / 4));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (head_dim == 128)
    hipLaunchKernelGGL(gqa_pack_kernel<128>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), num_tokens, num_kv_heads, slot_mapping,
                       static_cast<uint8_t*>(pool), num_pages);
  else
    hipLaunchKernelGGL(gqa_pack_kernel<64>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(k),
                       static_cast<const uint16_t*>(v), num_tokens, num_kv_heads, slot_mapping,
                       static_cast<uint8_t*>(pool), num_pages);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? ok() : fail(MQA_ERR_HIP, "gqa pack: %s", hipGetErrorString(e));
}

size_t mqa_gqa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t max_context, int32_t window, int32_t head_dim) {
  GqaArgs a{};
  size_t ws = 0;
  if (gqa_plan(batch, num_q_heads, num_kv_heads, max_context, window, head_dim, a, ws) != MQA_OK)
    return 0;
  return ws;
}

int mqa_gqa_decode_bf16(const void* q, float* out, const void* pool, int64_t num_pages,
                        int32_t num_kv_heads, int32_t head_dim, const int32_t* block_table,
                        int32_t max_pages, const int32_t* context_lens, int32_t max_context,
                        int32_t batch, int32_t num_q_heads, int32_t window, float softmax_scale,
                        void* workspace, size_t workspace_bytes, void* stream) {
  GqaArgs a{};
  size_t ws = 0;
  int rc = gqa_plan(batch, num_q_heads, num_kv_heads, max_context, window, head_dim, a, ws);
  if (rc) return rc;
  if (batch == 0) return ok();
  if (!q || !out || !pool || !block_table || !context_lens)
    return fail(MQA_ERR_INVALID, "NULL pointer");
  if (num_pages <= 0 || !aligned256(pool)) return fail(MQA_ERR_INVALID, "bad pool");
  if (max_pages < 1 || (int64_t)max_pages * 16 < max_context)
    return fail(MQA_ERR_INVALID, "max_pages %d cannot hold max_context %d", max_pages, max_context);
  if ((reinterpret_cast<uintptr_t>(q) & 15) || (reinterpret_cast<uintptr_t>(out) & 15))
    return fail(MQA_ERR_INVALID, "q and out must be 16-byte aligned");
  if (ws && (!workspace || workspace_bytes < ws))
    return fail(MQA_ERR_WORKSPACE, "workspace of %zu bytes needed", ws);
  if (!(softmax_scale >= 0.0f) ||
      (double)softmax_scale * 1.4426950408889634 > 3.4028234663852886e38)
    return fail(MQA_ERR_INVALID, "softmax_scale must be >= 0 and finite (scale * log2(e) in fp32)");
  const float scale = softmax_scale > 0.0f ? softmax_scale : 1.0f / sqrtf((float)head_dim);
  a.num_pages = num_pages;
  a.max_pages = max_pages;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)a.total_wgs), block(kGqaWaves * 64);
  float* wsf = static_cast<float*>(workspace);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* pp = static_cast<const uint8_t*>(pool);
  if (head_dim == 128)
    hipLaunchKernelGGL(gqa_decode_kernel<128>, grid, block, 0, s, a, qq, out, pp, block_table,
                       context_lens, wsf);
  else
    hipLaunchKernelGGL(gqa_decode_kernel<64>, grid, block, 0, s, a, qq, out, pp, block_table,
                       context_lens, wsf);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.nchunk > 1) {
    const dim3 mg((unsigned)(batch * num_kv_heads));
    if (head_dim == 128)
      hipLaunchKernelGGL(gqa_merge_kernel<128>, mg, dim3(256), 0, s, a, out, context_lens, wsf);
    else
      hipLaunchKernelGGL(gqa_merge_kernel<64>, mg, dim3(256), 0, s, a, out, context_lens, wsf);
    e = hipGetLastError();
  }
  return e == hipSuccess ? ok() : fail(MQA_ERR_HIP, "gqa decode: %s", hipGetErrorString(e));
}

}  // extern "C"
