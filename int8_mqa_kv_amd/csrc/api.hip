// C entry points of libmqa_kv: argument checks, launch planning, launches.
// Every check runs on the host before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mqa_kv.h"
#include "internal.hpp"

using namespace mqa;

namespace mqa {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return MQA_OK;
}

}  // namespace mqa

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(MQA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

namespace mqa {

int check_pool(const mqa_kv_pool* pool) {
  if (!pool) return fail(MQA_ERR_INVALID, "pool is NULL");
  if (pool->head_dim != 64 && pool->head_dim != 128)
    return fail(MQA_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", pool->head_dim);
  if (pool->num_pages <= 0) return fail(MQA_ERR_INVALID, "pool has %lld pages",
                                        (long long)pool->num_pages);
  if (!pool->base) return fail(MQA_ERR_INVALID, "pool base is NULL");
  if (!aligned(pool->base, 256)) return fail(MQA_ERR_INVALID, "pool base is not 256-byte aligned");
  if (pool->reserved != 0) return fail(MQA_ERR_INVALID, "pool.reserved must be 0");
  return MQA_OK;
}

}  // namespace mqa

namespace {

// Shape checks common to decode and append.
int check_attn_common(const void* q, mqa_dtype q_dtype, const float* out, const mqa_kv_pool* pool,
                      const int32_t* block_table, int32_t max_pages_per_seq,
                      const int32_t* context_lens, int32_t max_context, int32_t batch,
                      int32_t num_q_heads, int32_t num_layers, int32_t num_slots,
                      const int32_t* layer_slot, const int32_t* layer_window) {
  int rc = check_pool(pool);
  if (rc) return rc;
  if (q_dtype != MQA_F32 && q_dtype != MQA_BF16)
    return fail(MQA_ERR_UNSUPPORTED, "q dtype %d unsupported", (int)q_dtype);
  if (batch <= 0) return fail(MQA_ERR_INVALID, "batch must be > 0 (got %d)", batch);
  if (num_q_heads <= 0) return fail(MQA_ERR_INVALID, "num_q_heads must be > 0");
  if (num_layers <= 0) return fail(MQA_ERR_INVALID, "num_layers must be > 0");
  if (num_slots <= 0) return fail(MQA_ERR_INVALID, "num_slots must be > 0");
  if (max_pages_per_seq <= 0) return fail(MQA_ERR_INVALID, "max_pages_per_seq must be > 0");
  if (max_context <= 0) return fail(MQA_ERR_INVALID, "max_context must be > 0");
  if (max_context > MQA_MAX_CONTEXT)
    return fail(MQA_ERR_UNSUPPORTED, "max_context %d above %d", max_context, MQA_MAX_CONTEXT);
  if ((int64_t)max_pages_per_seq * kPageTokens < max_context)
    return fail(MQA_ERR_INVALID, "max_pages_per_seq*16 = %lld < max_context %d",
                (long long)max_pages_per_seq * kPageTokens, max_context);
  if (!q || !out || !block_table || !context_lens)
    return fail(MQA_ERR_INVALID, "q, out, block_table and context_lens must be non-NULL");
  if (!layer_slot || !layer_window)
    return fail(MQA_ERR_INVALID, "layer_slot and layer_window (host arrays) must be non-NULL");
  if (!aligned(q, 16) || !aligned(out, 16))
    return fail(MQA_ERR_INVALID, "q and out must be 16-byte aligned");
  if ((int64_t)num_slots * batch * max_pages_per_seq > INT64_C(1) << 40)
    return fail(MQA_ERR_INVALID, "block table too large");
  for (int l = 0; l < num_layers; ++l) {
    if (layer_slot[l] < 0 || layer_slot[l] >= num_slots)
      return fail(MQA_ERR_INVALID, "layer_slot[%d] = %d outside [0, %d)", l, layer_slot[l],
                  num_slots);
    if (layer_window[l] < 0)
      return fail(MQA_ERR_INVALID, "layer_window[%d] = %d is negative", l, layer_window[l]);
  }
  return MQA_OK;
}

// A softmax scale the kernels can use: <= 0 (the default), or positive with
// scale * log2(e) finite in fp32.  NaN and infinities are refused.
bool scale_ok(float softmax_scale) {
  return softmax_scale <= 0.0f ||
         (softmax_scale > 0.0f && (double)softmax_scale * 1.4426950408889634 <= 3.4028234663852886e38);
}

float scale_log2_of(float softmax_scale, int head_dim) {
  const double s = softmax_scale > 0.0f ? (double)softmax_scale : 1.0 / sqrt((double)head_dim);
  return (float)(s * 1.4426950408889634);
}

// ---------------------------------------------------------------------------
// Decode planning
// ---------------------------------------------------------------------------
struct DecodePlan {
  DecodeArgs args;
  int nrt = 2;
  int waves = kDecodeWaves;   // wavefronts per workgroup
  size_t ws_bytes = 0;        // partial records + arrival counters
  int rc = MQA_OK;
};

// Decode tuning overrides (0 = the planner decides), process-wide.  They start
// from MQA_DECODE_WAVES (4 or 8), MQA_DECODE_ROWS (8, 16 or 32) and
// MQA_DECODE_TARGET_WGS, and mqa_decode_tuning() replaces them.  Results do
// not depend on them beyond rounding order.  Each value is one atomic, so a
// change racing with a call is no data race; that call plans with the old or
// the new value of each.
struct DecodeTuning {
  std::atomic<int> waves{0}, rows{0}, target_wgs{0};
};
DecodeTuning& tuning() {
  static DecodeTuning t;
  static std::once_flag once;
  std::call_once(once, [] {
    auto env = [](const char* name) {
      const char* e = getenv(name);
      return e ? atoi(e) : 0;
    };
    const int w = env("MQA_DECODE_WAVES"), r = env("MQA_DECODE_ROWS"), g = env("MQA_DECODE_TARGET_WGS");
    t.waves = (w == kDecodeWaves || w == kDecodeWavesSmall) ? w : 0;
    t.rows = (r == 8 || r == 16 || r == 32) ? r : 0;
    t.target_wgs = g > 0 ? g : 0;
  });
  return t;
}

// Workgroups of kDecodeWaves wavefronts the planner aims for: one per compute
// unit of the 256 (twice as many of the four-wavefront shape).
int target_workgroups() {
  const int g = tuning().target_wgs;
  return g > 0 ? g : 256;
}
int decode_rows_override() { return tuning().rows; }

// Query rows per row block.  32 rows (two 16-row tiles per wavefront) read
// each page once for the most rows and cost the least vector work per (row,
// key).  When every sequence's key range is short (at most 128 pages: the
// 1024-token window, short contexts), a launch is bound by latency instead:
// its keys are split into few chunks whose partial results must be handed
// between workgroups.  There, 16-row blocks double the workgroups per page
// (the second reads the pages from L2), halve the chunks each range needs and
// the size of every partial record, and shorten the handoff.
// fp32 queries are carried as two fp16 terms per element, which leaves the
// registers for one 16-row tile per wavefront: 16-row blocks (or 8).
int decode_rows(int num_q_heads, int num_layers, int64_t max_span_pages, int64_t items32,
                bool q_f32) {
  int rows = decode_rows_override();
  if (rows == 0)
    rows = (num_q_heads > 16 && max_span_pages <= 128 && 2 * items32 <= target_workgroups())
               ? 16 : kRowsPerBlock;
  if (q_f32) return std::min(rows, 16);
  if (num_layers * ((num_q_heads + rows - 1) / rows) > kMaxRowBlocks) rows = kRowsPerBlock;
  return rows;
}

DecodePlan plan_decode(int32_t batch, int32_t num_q_heads, int32_t num_layers,
                       const int32_t* layer_slot, const int32_t* layer_window,
                       int32_t max_context, int32_t head_dim, bool q_f32, int waves) {
  DecodePlan p;
  p.waves = waves;
  DecodeArgs& a = p.args;
  memset(&a, 0, sizeof a);
  // groups of layers reading one slot with one window, in first-seen order
  std::vector<std::pair<int, int>> keys;
  std::vector<std::vector<int>> members;
  for (int l = 0; l < num_layers; ++l) {
    const std::pair<int, int> k{layer_slot[l], layer_window[l]};
    auto it = std::find(keys.begin(), keys.end(), k);
    if (it == keys.end()) {
      keys.push_back(k);
      members.push_back({l});
    } else {
      members[it - keys.begin()].push_back(l);
    }
  }
  if ((int)keys.size() > kMaxGroups) {
    p.rc = fail(MQA_ERR_UNSUPPORTED, "%d (slot, window) groups in one call; at most %d",
                (int)keys.size(), kMaxGroups);
    return p;
  }

  // Pages a sequence can span in each group (a window that does not start on
  // a page boundary touches one page more).
  const int64_t ctx_pages = (max_context + kPageTokens - 1) / kPageTokens;
  std::vector<int64_t> max_np(keys.size());
  int64_t span = 0;
  for (size_t g = 0; g < keys.size(); ++g) {
    const int w = keys[g].second;
    max_np[g] = w > 0 ? std::min<int64_t>((w + kPageTokens - 1) / kPageTokens + 1, ctx_pages)
                      : ctx_pages;
    span = std::max(span, max_np[g]);
  }
  const int64_t items32 =
      (int64_t)num_layers * ((num_q_heads + kRowsPerBlock - 1) / kRowsPerBlock) * batch;
  const int rows = decode_rows(num_q_heads, num_layers, span, items32, q_f32);
  p.nrt = std::min(rows, (int)num_q_heads) <= 16 ? 1 : 2;
  const int head_blocks = (num_q_heads + rows - 1) / rows;
  if (num_layers * head_blocks > kMaxRowBlocks) {
    p.rc = fail(MQA_ERR_UNSUPPORTED, "%d row blocks (layers x ceil(heads/%d)) in one call; at most %d",
                num_layers * head_blocks, rows, kMaxRowBlocks);
    return p;
  }

  // The work of all items, an item being one row block of one sequence.
  int64_t items = 0, work = 0;
  for (size_t g = 0; g < keys.size(); ++g) {
    const int64_t n = (int64_t)members[g].size() * head_blocks * batch;
    items += n;
    work += n * max_np[g];
  }
  static_assert((MQA_MAX_CONTEXT / kPageTokens + 1 + 255) / 256 <= kMaxDecodeChunks,
                "every wavefront's pages fit one register of page ids at the largest context");
  // Chunks per item: a share of the target workgroup count in proportion to
  // the item's span, so that one round of workgroups covers the launch with
  // equal work per workgroup and none left idle; at least enough chunks that
  // no wavefront takes more than 64 pages (one register of page ids).
  const int64_t target = std::max<int64_t>(target_workgroups() * (kDecodeWaves / waves), items);
  std::vector<int64_t> nchunk(keys.size());
  for (size_t g = 0; g < keys.size(); ++g) {
    const int64_t share = target * max_np[g] / std::max<int64_t>(work, 1);
    const int64_t need = (max_np[g] + 64 * waves - 1) / (64 * waves);
    // at most kMaxDecodeChunks (under MQA_MAX_CONTEXT, need stays below it)
    nchunk[g] = std::min<int64_t>(std::max<int64_t>({1, share, need}), kMaxDecodeChunks);
  }

  int rb = 0;
  int64_t wg = 0, ws = 0, merges = 0;
  bool split = false;
  for (size_t g = 0; g < keys.size(); ++g) {
    DecodeGroup& G = a.groups[g];
    G.slot = keys[g].first;
    G.window = keys[g].second;
    // the first group reading a slot stores that slot's current token
    G.writes_new_kv = 1;
    for (size_t h = 0; h < g; ++h)
      if (keys[h].first == G.slot) G.writes_new_kv = 0;
    G.first_rb = rb;
    for (int l : members[g])
      for (int hb = 0; hb < head_blocks; ++hb) {
        a.rbs[rb].layer = l;
        a.rbs[rb].head0 = hb * rows;
        a.rbs[rb].nrows = std::min(rows, num_q_heads - hb * rows);
        ++rb;
      }
    G.num_rb = rb - G.first_rb;
    G.nchunk = (int)nchunk[g];
    G.rb_recip = recip_of((uint32_t)G.num_rb);
    G.ch_recip = recip_of((uint32_t)G.nchunk);
    G.wg_begin = (int)wg;
    G.ws_begin = (int)ws;
    G.merge_begin = (int)merges;
    wg += (int64_t)G.num_rb * batch * G.nchunk;
    if (G.nchunk > 1) split = true;
    ws += (int64_t)G.num_rb * batch * G.nchunk;
    merges += (int64_t)G.num_rb * batch;
  }
  // one dispatch holds at most 2^32 - 1 work-items (the grid is padded to a multiple of 8)
  if ((wg + 8) * waves * 64 > INT64_C(0xFFFFFFFF) || ws > (INT64_C(1) << 30)) {
    p.rc = fail(MQA_ERR_UNSUPPORTED, "launch too large: %lld workgroups", (long long)wg);
    return p;
  }
  // Page loads go non-temporal where keeping the pages in the L2 buys
  // nothing: a slot that one row block reads, or one whose readers each walk
  // at most 8 pages per wavefront (they all reach a page within a few blocks
  // of one another).  Measured: one reader 4-7 % faster, two readers of short
  // windowed ranges 5 % faster; two or three readers over 16k keys 3-10 %
  // slower, since the later readers then miss the L2.
  for (size_t g = 0; g < keys.size(); ++g) {
    int readers = 0;
    int64_t walk = 0;  // pages per wavefront, the longest among the slot's groups
    for (size_t h = 0; h < keys.size(); ++h)
      if (keys[h].first == keys[g].first) {
        readers += a.groups[h].num_rb;
        walk = std::max<int64_t>(walk, (max_np[h] + nchunk[h] * waves - 1) / (nchunk[h] * waves));
      }
    a.groups[g].nontemporal = readers == 1 || walk <= 8;
  }
  a.num_groups = (int)keys.size();
  a.total_wgs = (int)wg;
  a.total_merge = (int)merges;
  if (split) {
    // the fixed counter prefix, then the partial records
    if (merges * waves > kDecodeCounters) {
      p.rc = fail(MQA_ERR_UNSUPPORTED,
                  "%lld (row block, sequence) pairs with split contexts in one call; at most %lld",
                  (long long)merges, (long long)(kDecodeCounters / waves));
      return p;
    }
    p.ws_bytes = (size_t)(kCounterWords + ws * ws_record_floats(head_dim)) * sizeof(float);
  }
  return p;
}

// The workgroup shape of a launch.  Eight wavefronts per workgroup, one
// workgroup per CU, unless that plan leaves more than 15 % of the CUs idle
// (few items, each split into whole chunks) while already splitting every
// item into at least two chunks, and four-wavefront workgroups, two per CU,
// fill at least 10 % more of the slots with at most 8 chunks per item (the
// last arrival folds every chunk's record).  An item the eight-wavefront plan
// keeps whole needs no handoff between workgroups; splitting it to fill the
// chip measured slower (short ranges are bound by latency, not by the loop).
DecodePlan plan_decode_auto(int32_t batch, int32_t num_q_heads, int32_t num_layers,
                            const int32_t* layer_slot, const int32_t* layer_window,
                            int32_t max_context, int32_t head_dim, bool q_f32) {
  const int forced_waves = tuning().waves;
  if (forced_waves)
    return plan_decode(batch, num_q_heads, num_layers, layer_slot, layer_window, max_context,
                       head_dim, q_f32, forced_waves);
  DecodePlan p8 = plan_decode(batch, num_q_heads, num_layers, layer_slot, layer_window,
                              max_context, head_dim, q_f32, kDecodeWaves);
  if (p8.rc) return p8;
  const double slots = target_workgroups();
  const double fill8 = p8.args.total_wgs / slots;
  if (fill8 >= 0.85) return p8;
  for (int g = 0; g < p8.args.num_groups; ++g)
    if (p8.args.groups[g].nchunk < 2) return p8;
  DecodePlan p4 = plan_decode(batch, num_q_heads, num_layers, layer_slot, layer_window,
                              max_context, head_dim, q_f32, kDecodeWavesSmall);
  if (p4.rc) {
    ok();  // the eight-wavefront plan stands; clear the other's message
    return p8;
  }
  int max_chunks = 0;
  for (int g = 0; g < p4.args.num_groups; ++g) max_chunks = std::max(max_chunks, p4.args.groups[g].nchunk);
  const double fill4 = p4.args.total_wgs / (slots * (kDecodeWaves / kDecodeWavesSmall));
  return (max_chunks <= 8 && fill4 <= 1.0 && fill4 >= fill8 + 0.10) ? p4 : p8;
}

}  // namespace

extern "C" {

int mqa_abi_version(void) { return MQA_KV_ABI_VERSION; }

const char* mqa_last_error(void) { return g_last_error.c_str(); }

size_t mqa_page_bytes(int32_t head_dim) {
  return (head_dim == 64 || head_dim == 128) ? (size_t)page_bytes(head_dim) : 0;
}

int64_t mqa_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                               int32_t dtype_bytes) {
  if (num_layers < 0 || num_kv_heads < 0 || head_dim < 0 || dtype_bytes < 0) return -1;
  return INT64_C(2) * num_layers * num_kv_heads * head_dim * dtype_bytes;
}

int mqa_page_offset(int32_t head_dim, int32_t token, int32_t channel, int32_t which,
                    int64_t* offset) {
  if (head_dim != 64 && head_dim != 128)
    return fail(MQA_ERR_UNSUPPORTED, "head_dim %d unsupported", head_dim);
  if (token < 0 || token >= kPageTokens) return fail(MQA_ERR_INVALID, "token %d not in [0,16)", token);
  if (!offset) return fail(MQA_ERR_INVALID, "offset is NULL");
  if (which == 0 || which == 1) {
    if (channel < 0 || channel >= head_dim)
      return fail(MQA_ERR_INVALID, "channel %d not in [0,%d)", channel, head_dim);
    *offset = which == 0 ? k_code_offset(head_dim, token, channel)
                         : v_code_offset(head_dim, token, channel);
  } else if (which == 2 || which == 3) {
    *offset = which == 2 ? k_scale_offset(head_dim, token) : v_scale_offset(head_dim, token);
  } else {
    return fail(MQA_ERR_INVALID, "which = %d not in {0,1,2,3}", which);
  }
  return ok();
}

int kv_pack_int8(const void* k, const void* v, mqa_dtype src_dtype, int64_t num_tokens,
                 int64_t row_stride, const int64_t* slot_mapping, const mqa_kv_pool* pool,
                 void* stream) {
  int rc = check_pool(pool);
  if (rc) return rc;
  if (src_dtype != MQA_F32 && src_dtype != MQA_BF16)
    return fail(MQA_ERR_UNSUPPORTED, "source dtype %d unsupported", (int)src_dtype);
  if (num_tokens < 0) return fail(MQA_ERR_INVALID, "num_tokens is negative");
  if (num_tokens > MQA_PACK_MAX_TOKENS)
    return fail(MQA_ERR_UNSUPPORTED, "num_tokens %lld above %d per call", (long long)num_tokens,
                MQA_PACK_MAX_TOKENS);
  if (num_tokens == 0) return ok();
  if (row_stride < pool->head_dim)
    return fail(MQA_ERR_INVALID, "row_stride %lld < head_dim %d", (long long)row_stride,
                pool->head_dim);
  if (!k || !v || !slot_mapping) return fail(MQA_ERR_INVALID, "k, v and slot_mapping must be non-NULL");
  const size_t esz = src_dtype == MQA_BF16 ? 2 : 4;
  if (!aligned(k, esz) || !aligned(v, esz) || !aligned(slot_mapping, 8))
    return fail(MQA_ERR_INVALID, "misaligned k, v or slot_mapping");
  hipError_t e = launch_pack(pool->head_dim, src_dtype == MQA_BF16, k, v, num_tokens, row_stride,
                             slot_mapping, static_cast<uint8_t*>(pool->base), pool->num_pages,
                             static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "kv_pack_int8 launch");
  return ok();
}

size_t mqa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_layers,
                                  const int32_t* layer_slot, const int32_t* layer_window,
                                  int32_t max_context, int32_t head_dim, mqa_dtype q_dtype) {
  if (batch <= 0 || num_q_heads <= 0 || num_layers <= 0 || max_context <= 0 ||
      max_context > MQA_MAX_CONTEXT || !layer_slot ||
      !layer_window || (head_dim != 64 && head_dim != 128) ||
      (q_dtype != MQA_F32 && q_dtype != MQA_BF16))
    return 0;
  for (int l = 0; l < num_layers; ++l)
    if (layer_slot[l] < 0 || layer_window[l] < 0) return 0;
  DecodePlan p = plan_decode_auto(batch, num_q_heads, num_layers, layer_slot, layer_window,
                                  max_context, head_dim, q_dtype == MQA_F32);
  return p.rc ? 0 : p.ws_bytes;
}

int mqa_decode_tuning(int32_t waves, int32_t rows, int32_t target_wgs) {
  if (waves != 0 && waves != kDecodeWaves && waves != kDecodeWavesSmall)
    return fail(MQA_ERR_INVALID, "waves %d: 0, %d or %d", waves, kDecodeWavesSmall, kDecodeWaves);
  if (rows != 0 && rows != 8 && rows != 16 && rows != 32)
    return fail(MQA_ERR_INVALID, "rows %d: 0, 8, 16 or 32", rows);
  if (target_wgs < 0) return fail(MQA_ERR_INVALID, "target_wgs %d < 0", target_wgs);
  DecodeTuning& t = tuning();
  t.waves = waves;
  t.rows = rows;
  t.target_wgs = target_wgs;
  return ok();
}

}  // extern "C"

namespace {

// Supplies the workspace of a decode call from somewhere other than the
// caller (the static scratch of mqa_decode_step_noalloc): called after every
// host check has passed and before the launch, with the bytes the plan needs
// (0 if none); sets *ws and returns MQA_OK, or a status that ends the call.
typedef int (*WorkspaceSource)(size_t need, void** ws, hipStream_t stream);

// Shared by mqa_decode_attn, mqa_decode_step and mqa_decode_step_noalloc.
int decode_common(const void* q, mqa_dtype q_dtype, float* out, const void* k_new,
                  const void* v_new, NewKV nk, const mqa_kv_pool* pool,
                  const int32_t* block_table, int32_t max_pages_per_seq,
                  const int32_t* context_lens, int32_t max_context, int32_t batch,
                  int32_t num_q_heads, int32_t num_layers, int32_t num_slots,
                  const int32_t* layer_slot, const int32_t* layer_window, float softmax_scale,
                  void* workspace, size_t workspace_bytes, void* stream, const char* what,
                  WorkspaceSource source = nullptr) {
  int rc = check_attn_common(q, q_dtype, out, pool, block_table, max_pages_per_seq, context_lens,
                             max_context, batch, num_q_heads, num_layers, num_slots, layer_slot,
                             layer_window);
  if (rc) return rc;
  if (!scale_ok(softmax_scale))
    return fail(MQA_ERR_INVALID, "softmax_scale %g is not a usable number", (double)softmax_scale);
  DecodePlan p = plan_decode_auto(batch, num_q_heads, num_layers, layer_slot, layer_window,
                                  max_context, pool->head_dim, q_dtype == MQA_F32);
  if (p.rc) return p.rc;
  if (source) {
    rc = source(p.ws_bytes, &workspace, static_cast<hipStream_t>(stream));
    if (rc) return rc;
    workspace_bytes = p.ws_bytes;
  }
  if (p.ws_bytes > 0) {
    if (!workspace || workspace_bytes < p.ws_bytes)
      return fail(MQA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", p.ws_bytes,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(MQA_ERR_INVALID, "workspace not 256-byte aligned");
  }
  DecodeArgs& a = p.args;
  a.num_pages = pool->num_pages;
  a.max_pages = max_pages_per_seq;
  a.max_context = max_context;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.scale_log2 = scale_log2_of(softmax_scale, pool->head_dim);
  DecodePtrs ptrs;
  ptrs.q = q;
  ptrs.out = out;
  ptrs.pool = static_cast<uint8_t*>(pool->base);
  ptrs.block_table = block_table;
  ptrs.context_lens = context_lens;
  ptrs.ws = p.ws_bytes ? static_cast<float*>(workspace) : nullptr;
  ptrs.k_new = k_new;
  ptrs.v_new = v_new;
  hipError_t e = launch_decode(pool->head_dim, q_dtype == MQA_F32, p.nrt, p.waves, nk, a, ptrs,
                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, what);
  return ok();
}

}  // namespace

extern "C" {

int mqa_decode_attn(const void* q, mqa_dtype q_dtype, float* out, const mqa_kv_pool* pool,
                    const int32_t* block_table, int32_t max_pages_per_seq,
                    const int32_t* context_lens, int32_t max_context, int32_t batch,
                    int32_t num_q_heads, int32_t num_layers, int32_t num_slots,
                    const int32_t* layer_slot, const int32_t* layer_window, float softmax_scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return decode_common(q, q_dtype, out, nullptr, nullptr, NewKV::kNone, pool, block_table,
                       max_pages_per_seq, context_lens, max_context, batch, num_q_heads,
                       num_layers, num_slots, layer_slot, layer_window, softmax_scale, workspace,
                       workspace_bytes, stream, "mqa_decode_attn launch");
}

int mqa_decode_step(const void* q, mqa_dtype q_dtype, float* out, const void* k_new,
                    const void* v_new, mqa_dtype kv_dtype, const mqa_kv_pool* pool,
                    const int32_t* block_table, int32_t max_pages_per_seq,
                    const int32_t* context_lens, int32_t max_context, int32_t batch,
                    int32_t num_q_heads, int32_t num_layers, int32_t num_slots,
                    const int32_t* layer_slot, const int32_t* layer_window, float softmax_scale,
                    void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_dtype != MQA_F32 && kv_dtype != MQA_BF16)
    return fail(MQA_ERR_UNSUPPORTED, "k_new/v_new dtype %d unsupported", (int)kv_dtype);
  if (!k_new || !v_new) return fail(MQA_ERR_INVALID, "k_new and v_new must be non-NULL");
  const size_t esz = kv_dtype == MQA_BF16 ? 2 : 4;
  if (!aligned(k_new, esz) || !aligned(v_new, esz))
    return fail(MQA_ERR_INVALID, "misaligned k_new or v_new");
  return decode_common(q, q_dtype, out, k_new, v_new,
                       kv_dtype == MQA_BF16 ? NewKV::kBf16 : NewKV::kF32, pool, block_table,
                       max_pages_per_seq, context_lens, max_context, batch, num_q_heads,
                       num_layers, num_slots, layer_slot, layer_window, softmax_scale, workspace,
                       workspace_bytes, stream, "mqa_decode_step launch");
}

int mqa_append_attn(const void* q, mqa_dtype q_dtype, float* out, const mqa_kv_pool* pool,
                    const int32_t* block_table, int32_t max_pages_per_seq,
                    const int32_t* context_lens, const int32_t* cu_q_lens, int32_t max_context,
                    int32_t max_q_len, int32_t total_q, int32_t batch, int32_t num_q_heads,
                    int32_t num_layers, int32_t num_slots, const int32_t* layer_slot,
                    const int32_t* layer_window, float softmax_scale, void* stream) {
  int rc = check_attn_common(q, q_dtype, out, pool, block_table, max_pages_per_seq, context_lens,
                             max_context, batch, num_q_heads, num_layers, num_slots, layer_slot,
                             layer_window);
  if (rc) return rc;
  if (!cu_q_lens) return fail(MQA_ERR_INVALID, "cu_q_lens must be non-NULL");
  if (max_q_len <= 0) return fail(MQA_ERR_INVALID, "max_q_len must be > 0");
  if (total_q <= 0) return fail(MQA_ERR_INVALID, "total_q must be > 0");
  if (!scale_ok(softmax_scale))
    return fail(MQA_ERR_INVALID, "softmax_scale %g is not a usable number", (double)softmax_scale);
  if (num_layers > kMaxLayers)
    return fail(MQA_ERR_UNSUPPORTED, "%d layers in one append call; at most %d", num_layers,
                kMaxLayers);
  AppendArgs a;
  memset(&a, 0, sizeof a);
  const int head_blocks = (num_q_heads + kRowsPerBlock - 1) / kRowsPerBlock;
  const int token_blocks = (max_q_len + kAppendWaves - 1) / kAppendWaves;
  const int64_t total = (int64_t)num_layers * batch * head_blocks * token_blocks;
  // one dispatch holds at most 2^32 - 1 work-items (the grid is padded to a multiple of 8)
  if ((total + 8) * kAppendWaves * 64 > INT64_C(0xFFFFFFFF))
    return fail(MQA_ERR_UNSUPPORTED, "launch too large: %lld workgroups", (long long)total);
  // layers ordered by slot, so layers sharing a slot run back to back
  std::vector<int> order(num_layers);
  for (int l = 0; l < num_layers; ++l) order[l] = l;
  std::stable_sort(order.begin(), order.end(),
                   [&](int x, int y) { return layer_slot[x] < layer_slot[y]; });
  for (int l = 0; l < num_layers; ++l) {
    a.order[l] = order[l];
    a.layer_slot[l] = layer_slot[l];
    a.layer_window[l] = layer_window[l];
  }
  a.num_pages = pool->num_pages;
  a.max_pages = max_pages_per_seq;
  a.max_context = max_context;
  a.batch = batch;
  a.num_q_heads = num_q_heads;
  a.total_q = total_q;
  a.num_layers = num_layers;
  a.head_blocks = head_blocks;
  a.token_blocks = token_blocks;
  a.total_wgs = (int)total;
  a.tb_recip = recip_of((uint32_t)token_blocks);
  a.hb_recip = recip_of((uint32_t)head_blocks);
  a.layer_recip = recip_of((uint32_t)num_layers);
  a.scale_log2 = scale_log2_of(softmax_scale, pool->head_dim);
  const int nrt = num_q_heads <= 16 ? 1 : 2;
  AppendPtrs ptrs;
  ptrs.q = q;
  ptrs.out = out;
  ptrs.pool = static_cast<const uint8_t*>(pool->base);
  ptrs.block_table = block_table;
  ptrs.context_lens = context_lens;
  ptrs.cu_q_lens = cu_q_lens;
  hipError_t e = launch_append(pool->head_dim, q_dtype == MQA_F32, nrt, a, ptrs,
                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mqa_append_attn launch");
  return ok();
}

}  // extern "C"

extern "C" {

int mqa_hbm_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t sink_words,
                       void* stream) {
  if (!src || !sink) return fail(MQA_ERR_INVALID, "src and sink must be non-NULL");
  if (bytes <= 0 || bytes % 16 != 0)
    return fail(MQA_ERR_INVALID, "bytes = %lld: a positive multiple of 16", (long long)bytes);
  if (!aligned(src, 16) || !aligned(sink, 4))
    return fail(MQA_ERR_INVALID, "src must be 16-byte and sink 4-byte aligned");
  if (sink_words < MQA_PROBE_SINK_WORDS)
    return fail(MQA_ERR_INVALID, "sink_words %d < %d", sink_words, MQA_PROBE_SINK_WORDS);
  hipError_t e = launch_hbm_read(src, bytes, sink, MQA_PROBE_SINK_WORDS,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "mqa_hbm_read_probe launch");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// mqa_decode_step_noalloc: mqa_decode_step with its workspace in a static
// device array of this library (one copy per GPU, held until the process
// ends), for callers that cannot allocate device memory.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[MQA_DECODE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

// Per device: the address of that device's copy of `scratch` (the array's
// name is a host-side stand-in, never a device address) and whether its
// arrival counters have been cleared once.
struct StaticScratch {
  std::once_flag once;
  hipError_t err = hipSuccess;
  void* ptr = nullptr;
  std::atomic<bool> cleared{false};
};
StaticScratch g_static_scratch[kMaxDevices];

__global__ void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

// The workspace source of mqa_decode_step_noalloc.  The first call on a
// device looks up that device's copy of `scratch` (with the device current).
// The arrival counters at its head must start at zero; every decode call
// leaves them at zero again, so they are cleared by a fill kernel on the
// caller's stream before the first decode that uses them (again on every
// call made while the stream is being captured, so that a graph captured
// first still clears them before its decode when replayed).  A fill kernel,
// not hipMemsetAsync, so that the clear can sit in a captured graph.
int static_scratch_source(size_t need, void** ws, hipStream_t stream) {
  if (need > (size_t)MQA_DECODE_STATIC_SCRATCH_BYTES)
    return fail(MQA_ERR_WORKSPACE,
                "this launch needs %zu bytes of decode scratch; the static scratch of "
                "mqa_decode_step_noalloc holds %zu (use mqa_decode_step with a workspace)",
                need, (size_t)MQA_DECODE_STATIC_SCRATCH_BYTES);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(MQA_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  StaticScratch& s = g_static_scratch[dev];
  std::call_once(s.once, [&] { s.err = hipGetSymbolAddress(&s.ptr, HIP_SYMBOL(scratch)); });
  if (s.err != hipSuccess) return hip_fail(s.err, "hipGetSymbolAddress(scratch)");
  if (!s.ptr) return fail(MQA_ERR_HIP, "hipGetSymbolAddress(scratch) gave a null address");
  *ws = s.ptr;
  if (need == 0 || s.cleared.load(std::memory_order_acquire)) return MQA_OK;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return hip_fail(e, "hipStreamIsCapturing");
  hipLaunchKernelGGL(zero_words_kernel, dim3(1024), dim3(256), 0, stream,
                     static_cast<uint32_t*>(s.ptr), kCounterWords);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "clearing the static decode scratch");
  if (cap == hipStreamCaptureStatusNone) s.cleared.store(true, std::memory_order_release);
  return MQA_OK;
}

}  // namespace

extern "C" {

int mqa_decode_step_noalloc(const void* q, mqa_dtype q_dtype, float* out, const void* k_new,
                            const void* v_new, mqa_dtype kv_dtype, const mqa_kv_pool* pool,
                            const int32_t* block_table, int32_t max_pages_per_seq,
                            const int32_t* context_lens, int32_t max_context, int32_t batch,
                            int32_t num_q_heads, int32_t num_layers, int32_t num_slots,
                            const int32_t* layer_slot, const int32_t* layer_window,
                            float softmax_scale, void* stream) {
  static_assert(MQA_DECODE_STATIC_SCRATCH_BYTES > kCounterWords * sizeof(float),
                "the static scratch holds the arrival counters and partial records");
  if (kv_dtype != MQA_F32 && kv_dtype != MQA_BF16)
    return fail(MQA_ERR_UNSUPPORTED, "k_new/v_new dtype %d unsupported", (int)kv_dtype);
  if (!k_new || !v_new) return fail(MQA_ERR_INVALID, "k_new and v_new must be non-NULL");
  const size_t esz = kv_dtype == MQA_BF16 ? 2 : 4;
  if (!aligned(k_new, esz) || !aligned(v_new, esz))
    return fail(MQA_ERR_INVALID, "misaligned k_new or v_new");
  return decode_common(q, q_dtype, out, k_new, v_new,
                       kv_dtype == MQA_BF16 ? NewKV::kBf16 : NewKV::kF32, pool, block_table,
                       max_pages_per_seq, context_lens, max_context, batch, num_q_heads,
                       num_layers, num_slots, layer_slot, layer_window, softmax_scale, nullptr, 0,
                       stream, "mqa_decode_step_noalloc launch", static_scratch_source);
}

}  // extern "C"
