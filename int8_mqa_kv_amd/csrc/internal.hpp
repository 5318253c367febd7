// Internal interfaces between the C entry points (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace mqa {

constexpr int kAppendWaves = 8;     // wavefronts (tokens) per append workgroup
constexpr int kAppendRing = 4;      // two-page blocks in an append workgroup's ring
constexpr int kRowsPerBlock = 32;   // query rows (heads) one wavefront carries
constexpr int kMaxGroups = 24;      // (slot, window) groups per decode launch
constexpr int kMaxRowBlocks = 64;   // row blocks per decode launch
constexpr int kMaxLayers = 64;      // layers per append launch

// Rows of one layer that one wavefront carries: heads [head0, head0+nrows).
struct RowBlock {
  int32_t layer;
  int32_t head0;
  int32_t nrows;
};

// Row blocks of layers that read one KV slot with one window.  The workgroups
// of a group are ordered (sequence, chunk, row block) so that every row block
// reading the same pages runs back to back on one XCD and shares its L2.
struct DecodeGroup {
  int32_t slot;
  int32_t window;
  int32_t first_rb;
  int32_t num_rb;
  int32_t nchunk;          // chunks (workgroups) per row block and sequence, at most
  int32_t wg_begin;        // first flat workgroup of the group
  int32_t ws_begin;        // first workspace record of the group
  int32_t merge_begin;     // first arrival counter of the group (row blocks x batch before it)
  int32_t writes_new_kv;   // this group stores the slot's current token (first group of a slot)
  int32_t nontemporal;     // page loads bypass the caches' retention (nothing reuses them soon)
  uint32_t rb_recip;       // floor((2^32 - 1) / num_rb): division by num_rb (udiv_recip)
  uint32_t ch_recip;       // floor((2^32 - 1) / nchunk)
};

// x / d for x < 2^31 and d >= 1 given recip = floor((2^32 - 1) / d): the
// high half of x * recip undershoots x / d by at most one, which one
// correction step repairs.
MQA_HD inline uint32_t recip_of(uint32_t d) { return 0xFFFFFFFFu / d; }

struct DecodeArgs {
  int64_t num_pages;
  int32_t max_pages;
  int32_t max_context;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_groups;
  int32_t total_wgs;
  int32_t total_merge;  // row blocks x batch (one arrival counter each)
  float scale_log2;     // softmax scale * log2(e)
  DecodeGroup groups[kMaxGroups];
  RowBlock rbs[kMaxRowBlocks];
};

// Device buffers of a decode call (kernel parameters of their own, marked
// __restrict__, so that uniform reads of tables become scalar loads).
struct DecodePtrs {
  const void* q;
  float* out;
  uint8_t* pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* ws;            // partial records + arrival counters (split sequences only)
  const void* k_new;    // current token's K rows [num_slots][batch][D] (fused step) or null
  const void* v_new;
};

// The current token's K/V handed to the fused decode step.
enum class NewKV { kNone = 0, kBf16 = 1, kF32 = 2 };

struct AppendArgs {
  int64_t num_pages;
  int32_t max_pages;
  int32_t max_context;
  int32_t batch;
  int32_t num_q_heads;
  int32_t total_q;
  int32_t num_layers;
  int32_t head_blocks;     // ceil(num_q_heads / 32)
  int32_t token_blocks;    // ceil(max_q_len / kAppendWaves)
  int32_t total_wgs;
  uint32_t tb_recip, hb_recip, layer_recip;  // recip_of(token_blocks / head_blocks / num_layers)
  float scale_log2;
  // layers in launch order (grouped by slot); order[i] is a layer index
  int32_t order[kMaxLayers];
  int32_t layer_slot[kMaxLayers];
  int32_t layer_window[kMaxLayers];
};

struct AppendPtrs {
  const void* q;
  float* out;
  const uint8_t* pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  const int32_t* cu_q_lens;
};

// Status reporting shared by the C entry points: fail() records the message
// mqa_last_error() returns and passes the status code through; ok() clears it.
int fail(int code, const char* fmt, ...);
int ok();
}  // namespace mqa
struct mqa_kv_pool;
namespace mqa {
// Checks of a pool descriptor shared by the entry points that take one.
int check_pool(const mqa_kv_pool* pool);

hipError_t launch_pack(int D, bool bf16, const void* k, const void* v, int64_t num_tokens,
                       int64_t row_stride, const int64_t* slot_mapping, uint8_t* pool,
                       int64_t num_pages, hipStream_t stream);

hipError_t launch_decode(int D, bool q_f32, int nrt, int waves, NewKV new_kv, const DecodeArgs& a,
                         const DecodePtrs& p, hipStream_t stream);

hipError_t launch_append(int D, bool q_f32, int nrt, const AppendArgs& a, const AppendPtrs& p,
                         hipStream_t stream);

// Streaming read of `bytes` (a multiple of 16) by `groups` workgroups, each
// writing the XOR of its range's 32-bit words to sink[its index].
hipError_t launch_hbm_read(const void* src, int64_t bytes, uint32_t* sink, int groups,
                           hipStream_t stream);

// Decode workspace: a fixed prefix of 32-bit arrival counters, one per
// (row block, sequence, wavefront) of a call and each on a 128-byte line of
// its own (atomics to one line serialise), then one partial record per
// (row block, sequence, chunk) of a split sequence.  A record holds, for each
// (16-row tile, 16-channel tile) pair of the output, m[16], l[16] and
// acc[4][64] fp32 (acc in matrix-core operand order), so that one wavefront
// writes and reads its pairs with whole 256-byte accesses.  The counter
// prefix has the same size and place for every call shape, so calls of
// different shapes can share one workspace: each leaves its counters at zero
// and records never overwrite a counter.
constexpr int kPairFloats = 16 + 16 + 4 * 64;
constexpr int64_t ws_record_floats(int D) { return (int64_t)2 * (D / 16) * kPairFloats; }
constexpr int64_t kDecodeCounters = 65536;        // arrival counters per call, at most
constexpr int64_t kCounterStride = 32;            // 32-bit words per counter (128 bytes)
constexpr int64_t kCounterWords = kDecodeCounters * kCounterStride;  // 8 MiB prefix
constexpr int kDecodeWaves = 8;     // wavefronts per decode workgroup (one workgroup per CU)
constexpr int kDecodeWavesSmall = 4;  // the two-per-CU shape for launches with few items
constexpr int kDecodeRing = 2;      // blocks of two pages in flight per wavefront
constexpr int kMaxDecodeChunks = 2048;  // chunks of one item's key range, at most

}  // namespace mqa
