// Host-side memory management of the paged cache: the KV footprint of a
// layer map, and a page table that grows sequences page by page and recycles
// the pages of windowed (local) slots once no later step can read them.
//
// "Character.AI: inference optimization", section 03 (technique table): most
// layers attend locally with a horizon of 1024 and only 1 in 6 is global, and
// global layers share one KV cache.  A local slot therefore never needs more
// than its window of tokens, and a shared slot is stored once.  "Como funciona
// a inferência de IA", section "O que os servidores de inferência em produção
// ... fazem a respeito?", item 1: the cache lives in fixed-size blocks placed
// anywhere in memory, with a per-request table saying where each block is;
// so a block that falls out of every window can go straight back to a free
// list and serve another sequence.
//
// No GPU work here: nothing is launched and no device memory is touched.
#include <stdint.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "../../include/mqa_kv.h"
#include "internal.hpp"

namespace {

using mqa::fail;
using mqa::ok;
constexpr int kPage = MQA_PAGE_TOKENS;

// First token a step ending at `context` (with `new_tokens` query tokens, the
// last at context-1) can still read through a window W: the earliest query,
// at context-new_tokens, sees the W tokens ending at its own position.
int64_t first_readable(int64_t context, int64_t new_tokens, int32_t window) {
  if (window <= 0) return 0;
  return std::max<int64_t>(0, context - new_tokens + 1 - window);
}

}  // namespace

// Per sequence and slot: the page id of every logical page, -1 where none is
// held (logical page i holds tokens [16i, 16i+16)).  The held pages of a
// (slot, sequence) are always one run [lo, end): a step frees a prefix of the
// run and extends it at the end, so every call costs the pages it changes.
struct mqa_page_table {
  int32_t num_pages = 0, first_page = 0, num_slots = 0, batch = 0, max_pages = 0;
  int32_t invalid_page = -1;
  std::vector<int32_t> window;       // [num_slots]; 0: global
  std::vector<int32_t> free_ids;     // stack: the last freed page is reused first
  std::vector<int64_t> context;      // [batch]
  std::vector<int64_t> qfirst;       // [batch]: earliest query position of the last step
  std::vector<int32_t> ids;          // [num_slots][batch][max_pages]
  std::vector<int64_t> lo, end;      // [num_slots][batch]: the held run
  int64_t item(int slot, int seq) const { return (int64_t)slot * batch + seq; }
  int32_t* row(int slot, int seq) { return ids.data() + item(slot, seq) * max_pages; }
};

extern "C" {

int64_t mqa_kv_footprint_bytes(int32_t num_layers, const int32_t* layer_slot,
                               const int32_t* layer_window, int32_t num_kv_heads,
                               int32_t head_dim, int32_t code_bytes, int32_t scale_bytes,
                               int64_t context, int32_t page_tokens) {
  if (num_layers < 0 || num_kv_heads < 0 || head_dim < 0 || code_bytes < 0 || scale_bytes < 0 ||
      context < 0 || page_tokens < 0 || (num_layers > 0 && (!layer_slot || !layer_window)))
    return -1;
  // each distinct slot once, with the widest reach of the layers reading it
  std::vector<std::pair<int32_t, int32_t>> slots;  // (slot, window; 0 = global)
  for (int l = 0; l < num_layers; ++l) {
    if (layer_slot[l] < 0 || layer_window[l] < 0) return -1;
    auto it = std::find_if(slots.begin(), slots.end(),
                           [&](const std::pair<int32_t, int32_t>& s) { return s.first == layer_slot[l]; });
    if (it == slots.end()) {
      slots.push_back({layer_slot[l], layer_window[l]});
    } else if (it->second != 0) {
      it->second = layer_window[l] == 0 ? 0 : std::max(it->second, layer_window[l]);
    }
  }
  const int64_t per_token =
      INT64_C(2) * num_kv_heads * ((int64_t)head_dim * code_bytes + scale_bytes);
  int64_t tokens = 0;
  for (const auto& s : slots) {
    if (context == 0) continue;
    const int64_t lo = first_readable(context, 1, s.second);
    if (page_tokens == 0) {
      tokens += context - lo;
    } else {
      tokens += ((context - 1) / page_tokens - lo / page_tokens + 1) * page_tokens;
    }
  }
  return tokens * per_token;
}

int mqa_page_table_create(int32_t first_page, int32_t num_pages, int32_t num_slots,
                          const int32_t* slot_window, int32_t batch, int32_t max_pages,
                          int32_t invalid_page, mqa_page_table** out) {
  if (!out) return fail(MQA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (first_page < 0 || num_pages < 0 || (int64_t)first_page + num_pages > INT32_MAX)
    return fail(MQA_ERR_INVALID, "page range [%d, %d + %d) invalid", first_page, first_page,
                num_pages);
  if (num_slots <= 0 || batch <= 0 || max_pages <= 0)
    return fail(MQA_ERR_INVALID, "num_slots, batch and max_pages must be positive");
  if (!slot_window) return fail(MQA_ERR_INVALID, "slot_window is NULL");
  for (int s = 0; s < num_slots; ++s)
    if (slot_window[s] < 0) return fail(MQA_ERR_INVALID, "slot_window[%d] < 0", s);
  if (invalid_page >= first_page && invalid_page < first_page + num_pages)
    return fail(MQA_ERR_INVALID, "invalid_page %d lies in the managed range", invalid_page);
  if ((int64_t)num_slots * batch * max_pages > (INT64_C(1) << 31))
    return fail(MQA_ERR_UNSUPPORTED, "table too large");
  mqa_page_table* t = new (std::nothrow) mqa_page_table;
  if (!t) return fail(MQA_ERR_INVALID, "out of host memory");
  t->num_pages = num_pages;
  t->first_page = first_page;
  t->num_slots = num_slots;
  t->batch = batch;
  t->max_pages = max_pages;
  t->invalid_page = invalid_page;
  t->window.assign(slot_window, slot_window + num_slots);
  t->free_ids.resize(num_pages);
  for (int i = 0; i < num_pages; ++i) t->free_ids[i] = first_page + num_pages - 1 - i;
  t->context.assign(batch, 0);
  t->qfirst.assign(batch, 0);
  t->ids.assign((size_t)num_slots * batch * max_pages, -1);
  t->lo.assign((size_t)num_slots * batch, 0);
  t->end.assign((size_t)num_slots * batch, 0);
  *out = t;
  return ok();
}

int mqa_page_table_destroy(mqa_page_table* t) {
  delete t;
  return ok();
}

}  // extern "C"

namespace {

// Checks of one sequence's step; MQA_OK or a status with the message set.
int check_step(const mqa_page_table* t, int32_t seq, int64_t context, int32_t new_tokens) {
  if (seq < 0 || seq >= t->batch) return fail(MQA_ERR_INVALID, "seq %d not in [0, %d)", seq, t->batch);
  const int64_t prev = t->context[seq];
  if (context < prev)
    return fail(MQA_ERR_INVALID, "seq %d: context %lld below the sequence's %lld", seq,
                (long long)context, (long long)prev);
  if (context > (int64_t)t->max_pages * kPage)
    return fail(MQA_ERR_INVALID, "seq %d: context %lld exceeds max_pages * 16", seq,
                (long long)context);
  if (new_tokens < 1 || new_tokens > context)
    return fail(MQA_ERR_INVALID, "seq %d: new_tokens %d not in [1, context]", seq, new_tokens);
  // pages behind a window were recycled for good: the earliest query of a
  // step may not move back before that of the sequence's last step
  if (prev > 0 && context - new_tokens < t->qfirst[seq])
    return fail(MQA_ERR_INVALID, "seq %d: earliest query %lld precedes the last step's %lld", seq,
                (long long)(context - new_tokens), (long long)t->qfirst[seq]);
  return MQA_OK;
}

// Pages one sequence's step frees and takes.
void count_step(const mqa_page_table* t, int32_t seq, int64_t context, int32_t new_tokens,
                int64_t& to_free, int64_t& to_alloc) {
  const int64_t new_end = (context - 1) / kPage + 1;
  for (int s = 0; s < t->num_slots; ++s) {
    const int64_t k = t->item(s, seq);
    const int64_t new_lo = first_readable(context, new_tokens, t->window[s]) / kPage;
    to_free += std::max<int64_t>(0, std::min(new_lo, t->end[k]) - t->lo[k]);
    to_alloc += new_end - std::max(new_lo, t->end[k]);
  }
}

void free_behind(mqa_page_table* t, int32_t seq, int64_t context, int32_t new_tokens,
                 int32_t* block_table) {
  for (int s = 0; s < t->num_slots; ++s) {
    const int64_t k = t->item(s, seq);
    int32_t* r = t->row(s, seq);
    int32_t* out = block_table ? block_table + k * t->max_pages : nullptr;
    const int64_t new_lo = first_readable(context, new_tokens, t->window[s]) / kPage;
    const int64_t stop = std::min(new_lo, t->end[k]);
    for (int64_t i = t->lo[k]; i < stop; ++i) {
      t->free_ids.push_back(r[i]);
      r[i] = -1;
      if (out) out[i] = t->invalid_page;
    }
    t->lo[k] = std::max(t->lo[k], stop);
  }
}

void grow(mqa_page_table* t, int32_t seq, int64_t context, int32_t new_tokens,
          int32_t* block_table) {
  const int64_t prev = t->context[seq];
  const int64_t new_end = (context - 1) / kPage + 1;
  for (int s = 0; s < t->num_slots; ++s) {
    const int64_t k = t->item(s, seq);
    int32_t* r = t->row(s, seq);
    int32_t* out = block_table ? block_table + k * t->max_pages : nullptr;
    const int64_t new_lo = first_readable(context, new_tokens, t->window[s]) / kPage;
    const int64_t from = std::max(new_lo, t->end[k]);
    for (int64_t i = from; i < new_end; ++i) {
      r[i] = t->free_ids.back();
      t->free_ids.pop_back();
      if (out) out[i] = r[i];
    }
    if (t->lo[k] >= t->end[k]) t->lo[k] = from;  // the run was empty or wholly freed
    t->end[k] = std::max(t->end[k], new_end);
    // a sequence's first call writes its whole row (every other entry invalid)
    if (out && prev == 0)
      for (int64_t i = 0; i < t->max_pages; ++i)
        if (i < t->lo[k] || i >= t->end[k]) out[i] = t->invalid_page;
  }
  t->context[seq] = context;
  t->qfirst[seq] = context - new_tokens;
}

}  // namespace

extern "C" {

int mqa_page_table_advance(mqa_page_table* t, int32_t seq, int64_t context, int32_t new_tokens,
                           int32_t* block_table) {
  if (!t) return fail(MQA_ERR_INVALID, "page table is NULL");
  int rc = check_step(t, seq, context, new_tokens);
  if (rc != MQA_OK) return rc;
  // count first, change nothing unless the free list covers the growth (the
  // pages this call frees count: they serve its own new pages first)
  int64_t to_free = 0, to_alloc = 0;
  count_step(t, seq, context, new_tokens, to_free, to_alloc);
  if (to_alloc > (int64_t)t->free_ids.size() + to_free)
    return fail(MQA_ERR_UNSUPPORTED, "page pool exhausted: %lld pages needed, %lld free",
                (long long)to_alloc, (long long)(t->free_ids.size() + to_free));
  free_behind(t, seq, context, new_tokens, block_table);
  grow(t, seq, context, new_tokens, block_table);
  return ok();
}

int mqa_page_table_advance_all(mqa_page_table* t, const int64_t* context,
                               const int32_t* new_tokens, int32_t* block_table) {
  if (!t) return fail(MQA_ERR_INVALID, "page table is NULL");
  if (!context || !new_tokens) return fail(MQA_ERR_INVALID, "context or new_tokens is NULL");
  int64_t to_free = 0, to_alloc = 0;
  for (int32_t b = 0; b < t->batch; ++b) {
    if (new_tokens[b] == 0) continue;  // not stepping
    int rc = check_step(t, b, context[b], new_tokens[b]);
    if (rc != MQA_OK) return rc;
    count_step(t, b, context[b], new_tokens[b], to_free, to_alloc);
  }
  if (to_alloc > (int64_t)t->free_ids.size() + to_free)
    return fail(MQA_ERR_UNSUPPORTED, "page pool exhausted: %lld pages needed, %lld free",
                (long long)to_alloc, (long long)(t->free_ids.size() + to_free));
  // every sequence frees before any grows: the step's frees serve its growth
  for (int32_t b = 0; b < t->batch; ++b)
    if (new_tokens[b] != 0) free_behind(t, b, context[b], new_tokens[b], block_table);
  for (int32_t b = 0; b < t->batch; ++b)
    if (new_tokens[b] != 0) grow(t, b, context[b], new_tokens[b], block_table);
  return ok();
}

int mqa_page_table_release(mqa_page_table* t, int32_t seq, int32_t* block_table) {
  if (!t) return fail(MQA_ERR_INVALID, "page table is NULL");
  if (seq < 0 || seq >= t->batch) return fail(MQA_ERR_INVALID, "seq %d not in [0, %d)", seq, t->batch);
  for (int s = 0; s < t->num_slots; ++s) {
    const int64_t k = t->item(s, seq);
    int32_t* r = t->row(s, seq);
    int32_t* out = block_table ? block_table + k * t->max_pages : nullptr;
    for (int64_t i = t->lo[k]; i < t->end[k]; ++i) {
      t->free_ids.push_back(r[i]);
      r[i] = -1;
      if (out) out[i] = t->invalid_page;
    }
    t->lo[k] = t->end[k] = 0;
  }
  t->context[seq] = 0;
  t->qfirst[seq] = 0;
  return ok();
}

int64_t mqa_page_table_free_pages(const mqa_page_table* t) {
  return t ? (int64_t)t->free_ids.size() : -1;
}

int64_t mqa_page_table_held_pages(const mqa_page_table* t, int32_t seq, int32_t slot) {
  if (!t || seq < 0 || seq >= t->batch || slot < 0 || slot >= t->num_slots) return -1;
  const int64_t k = t->item(slot, seq);
  return t->end[k] - t->lo[k];
}

int mqa_page_table_slot_mapping(const mqa_page_table* t, int32_t seq, int32_t slot, int64_t start,
                                int32_t count, int64_t* out) {
  if (!t) return fail(MQA_ERR_INVALID, "page table is NULL");
  if (seq < 0 || seq >= t->batch || slot < 0 || slot >= t->num_slots)
    return fail(MQA_ERR_INVALID, "(seq %d, slot %d) out of range", seq, slot);
  if (count < 0 || (count > 0 && !out)) return fail(MQA_ERR_INVALID, "bad count or out");
  const int32_t* r = const_cast<mqa_page_table*>(t)->row(slot, seq);
  for (int32_t k = 0; k < count; ++k) {
    const int64_t pos = start + k;
    const int64_t i = pos / kPage;
    if (pos < 0 || i >= t->max_pages || r[i] < 0)
      return fail(MQA_ERR_INVALID, "token %lld of (seq %d, slot %d) has no page", (long long)pos,
                  seq, slot);
  }
  for (int32_t k = 0; k < count; ++k) {
    const int64_t pos = start + k;
    out[k] = (int64_t)r[pos / kPage] * kPage + pos % kPage;
  }
  return ok();
}

}  // extern "C"
