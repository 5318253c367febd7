// Internal interfaces between the C entry points (api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.hpp"

namespace mqa {

constexpr int kAttnWaves = 4;       // wavefronts per attention workgroup
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
  int32_t pages_per_wave;  // even
  int32_t nchunk;          // chunks per sequence planned for max_context
  int32_t wg_begin;        // first flat workgroup of the group
  int32_t ws_begin;        // first workspace record of the group
  int32_t merge_begin;     // first merge workgroup of the group (row blocks x batch before it)
  int32_t waves;           // wavefronts per decode workgroup
};

struct DecodeArgs {
  int64_t num_pages;
  int32_t max_pages;
  int32_t max_context;
  int32_t batch;
  int32_t num_q_heads;
  int32_t num_groups;
  int32_t total_wgs;
  int32_t total_merge;  // row blocks x batch
  float scale_log2;     // softmax scale * log2(e)
  DecodeGroup groups[kMaxGroups];
  RowBlock rbs[kMaxRowBlocks];
};

// Device buffers of a decode call (kernel parameters of their own, marked
// __restrict__, so that uniform reads of tables become scalar loads).
struct DecodePtrs {
  const void* q;
  float* out;
  const uint8_t* pool;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* ws;            // partial records of sequences split into several chunks
};

struct AppendArgs {
  int64_t num_pages;
  int32_t max_pages;
  int32_t max_context;
  int32_t batch;
  int32_t num_q_heads;
  int32_t total_q;
  int32_t num_layers;
  int32_t head_blocks;     // ceil(num_q_heads / 32)
  int32_t token_blocks;    // ceil(max_q_len / kAttnWaves)
  int32_t total_wgs;
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

hipError_t launch_pack(int D, bool bf16, const void* k, const void* v, int64_t num_tokens,
                       int64_t row_stride, const int64_t* slot_mapping, uint8_t* pool,
                       int64_t num_pages, hipStream_t stream);

hipError_t launch_decode(int D, bool q_f32, int nrt, int waves, int ring, const DecodeArgs& a,
                         const DecodePtrs& p, bool need_merge, hipStream_t stream);

hipError_t launch_append(int D, bool q_f32, int nrt, const AppendArgs& a, const AppendPtrs& p,
                         hipStream_t stream);

// Decode workspace record: m[32], l[32], acc[32][D] fp32.
constexpr int64_t ws_record_floats(int D) { return kRowsPerBlock * (D + 2); }

}  // namespace mqa
