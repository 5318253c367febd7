// Cross-turn prefix cache: K/V pages of earlier turns kept in host memory and
// restored into the paged pool when a new turn starts with a cached prefix.
//
// "Character.AI: inference optimization", section 04 (cache between turns):
// the attention KV of a dialogue is kept in host memory, in a tree-structured
// LRU cache indexed by a rolling hash of every prefix, so that a new message
// -- or a regeneration that shares only part of the history -- finds the
// longest cached prefix and only the rest is computed.  "Como funciona a
// inferência de IA", section "O que os servidores ... fazem a respeito?",
// item 3 (prefix caching): K/V of a shared opening are computed once.
//
// MI355X design: a node of the cache is one page (16 tokens) of one dialogue
// prefix, so the tree is a radix tree over pages; it owns one arena entry per
// KV slot whose page it holds (a windowed slot keeps only its last pages, so
// most nodes of a long dialogue hold the global slots alone), and a restored
// page lands in the pool as-is.  The entries live in a pinned host arena the
// caller owns; one page-copy kernel moves a
// whole batch of pages between the pool and the arena over the host link
// (pool -> host at the end of a turn, host -> pool at the start of the next),
// reading its list of (source, destination) offsets from a small command ring
// at the head of the arena.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/mqa_kv.h"
#include "internal.hpp"

namespace mqa {

// One wavefront per (source, destination) pair of byte offsets: `bytes`
// (a multiple of 16) from src + pairs[2i] to dst + pairs[2i+1].
__global__ __launch_bounds__(256) void page_copy_kernel(const uint8_t* __restrict__ src,
                                                        uint8_t* __restrict__ dst,
                                                        const int64_t* __restrict__ pairs, int n,
                                                        int bytes) {
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= n) return;
  const int lane = threadIdx.x & 63;
  const int64_t so = pairs[2 * i], dof = pairs[2 * i + 1];
  for (int off = lane * 16; off < bytes; off += 64 * 16)
    *reinterpret_cast<uint4*>(dst + dof + off) = *reinterpret_cast<const uint4*>(src + so + off);
}

}  // namespace mqa

namespace {

using mqa::fail;
using mqa::ok;
constexpr int kPage = MQA_PAGE_TOKENS;
constexpr int kRing = 4;                    // command regions in flight
constexpr int64_t kRingBytes = 64 * 1024;   // per region: 4096 (source, destination) pairs

// Rolling hash of a prefix, page by page: FNV-1a over the page's 16 token
// ids chained from the previous page's value, then a splitmix64 finaliser.
uint64_t chain_hash(uint64_t h, const int32_t* t) {
  for (int i = 0; i < kPage; ++i) {
    h ^= (uint32_t)t[i];
    h *= 0x100000001b3ull;
  }
  h ^= h >> 30;
  h *= 0xbf58476d1ce4e5b9ull;
  h ^= h >> 27;
  h *= 0x94d049bb133111ebull;
  h ^= h >> 31;
  return h;
}
constexpr uint64_t kHashSeed = 0xcbf29ce484222325ull;

struct Node {
  uint64_t hash = 0;
  uint64_t present = 0;        // slots whose page this node holds
  int32_t parent = -1;         // node of the previous page, -1 for a first page
  int32_t children = 0;
  int32_t prev = -1, next = -1;  // LRU list (head: most recent)
  uint32_t mark = 0;           // epoch stamp of the insert walking through it
  int32_t tokens[kPage];
  bool live = false;
};

}  // namespace

struct mqa_prefix_cache {
  uint8_t* arena = nullptr;      // host
  uint8_t* arena_dev = nullptr;  // the same memory as the GPU addresses it (null: host only)
  int64_t arena_bytes = 0;
  int32_t num_slots = 0, head_dim = 0, page_bytes = 0;
  int64_t entry_bytes = 0, entries_base = 0, capacity = 0;  // entries: one (page, slot) each
  std::vector<int32_t> window;
  std::vector<Node> nodes;
  std::vector<int32_t> slot_entry;   // [node][slot]: arena entry, -1 if not held
  std::vector<int32_t> free_nodes, free_entries;
  std::unordered_multimap<uint64_t, int32_t> index;
  int32_t head = -1, tail = -1;
  uint32_t epoch = 0;
  hipEvent_t ev[kRing] = {};
  bool ev_pending[kRing] = {};
  int next_region = 0;
  int64_t stats[6] = {};  // lookups, tokens asked, tokens matched, entries inserted, evicted, restored

  int64_t entry_off(int32_t e) const { return entries_base + (int64_t)e * entry_bytes; }
  int32_t& ent(int32_t n, int s) { return slot_entry[(size_t)n * num_slots + s]; }
  int32_t ent(int32_t n, int s) const { return slot_entry[(size_t)n * num_slots + s]; }

  void unlink(int32_t n) {
    Node& x = nodes[n];
    if (x.prev >= 0) nodes[x.prev].next = x.next; else head = x.next;
    if (x.next >= 0) nodes[x.next].prev = x.prev; else tail = x.prev;
    x.prev = x.next = -1;
  }
  void push_front(int32_t n) {
    Node& x = nodes[n];
    x.prev = -1;
    x.next = head;
    if (head >= 0) nodes[head].prev = n;
    head = n;
    if (tail < 0) tail = n;
  }
  void touch(int32_t n) {
    unlink(n);
    push_front(n);
  }
  // a path's nodes from leaf to root: every parent ends up more recent than
  // its children, so the least recent node is always a leaf
  void touch_path(const std::vector<int32_t>& path, size_t len) {
    for (size_t i = len; i-- > 0;) touch(path[i]);
  }
  int32_t find(uint64_t h, int32_t parent, const int32_t* t) const {
    auto r = index.equal_range(h);
    for (auto it = r.first; it != r.second; ++it) {
      const Node& x = nodes[it->second];
      if (x.parent == parent && memcmp(x.tokens, t, sizeof x.tokens) == 0) return it->second;
    }
    return -1;
  }
  void evict(int32_t n) {
    Node& x = nodes[n];
    unlink(n);
    auto r = index.equal_range(x.hash);
    for (auto it = r.first; it != r.second; ++it)
      if (it->second == n) {
        index.erase(it);
        break;
      }
    if (x.parent >= 0) --nodes[x.parent].children;
    for (int s = 0; s < num_slots; ++s)
      if (ent(n, s) >= 0) {
        free_entries.push_back(ent(n, s));
        ent(n, s) = -1;
        ++stats[4];
      }
    x.present = 0;
    x.live = false;
    free_nodes.push_back(n);
  }
  // at least `k` free entries, evicting least recent leaves not on the
  // current walk; false if the walk itself holds too much of the arena
  bool reserve(int64_t k) {
    while ((int64_t)free_entries.size() < k) {
      int32_t victim = -1;
      for (int32_t n = tail; n >= 0; n = nodes[n].prev)
        if (nodes[n].children == 0 && nodes[n].mark != epoch) {
          victim = n;
          break;
        }
      if (victim < 0) return false;
      evict(victim);
    }
    return true;
  }
  int32_t take_entry() {
    const int32_t e = free_entries.back();
    free_entries.pop_back();
    return e;
  }
  // the longest run of cached pages of tokens[0 .. 16*max_pages)
  void walk(const int32_t* tokens, int64_t max_pages, std::vector<int32_t>& path) const {
    path.clear();
    uint64_t h = kHashSeed;
    int32_t parent = -1;
    for (int64_t k = 0; k < max_pages; ++k) {
      h = chain_hash(h, tokens + k * kPage);
      const int32_t n = find(h, parent, tokens + k * kPage);
      if (n < 0) break;
      path.push_back(n);
      parent = n;
    }
  }
  // The longest P such that a step whose earliest query sits at token 16*P
  // finds every page it reads cached: all pages before it for a global slot
  // (a property of a prefix), the pages its window reaches for a windowed one.
  int64_t restorable(const std::vector<int32_t>& path) const {
    uint64_t gmask = 0;
    for (int s = 0; s < num_slots; ++s)
      if (window[s] == 0) gmask |= 1ull << s;
    int64_t P = (int64_t)path.size();
    for (int64_t k = 0; k < P; ++k)
      if ((nodes[path[k]].present & gmask) != gmask) {
        P = k;
        break;
      }
    // A windowed slot missing page m rules out every P' in (m, P]: their
    // windows start no later than P's and still end after m.  So the search
    // jumps to the highest missing page of the failing window.
    while (P > 0) {
      int64_t jump = P;
      for (int s = 0; s < num_slots; ++s) {
        if (window[s] == 0) continue;
        const int64_t lo = std::max<int64_t>(0, kPage * P + 1 - window[s]) / kPage;
        for (int64_t k = P; k-- > lo;)
          if (!(nodes[path[k]].present & (1ull << s))) {
            jump = std::min(jump, k);
            break;
          }
      }
      if (jump == P) break;
      P = jump;
    }
    return P;
  }

  // Copies through the command ring: pairs of (source, destination) offsets.
  int copy(const uint8_t* src, uint8_t* dst, const std::vector<int64_t>& pairs,
           hipStream_t stream) {
    const int64_t per = kRingBytes / 16;
    for (size_t i0 = 0; i0 < pairs.size() / 2; i0 += per) {
      const int n = (int)std::min<int64_t>(per, (int64_t)pairs.size() / 2 - i0);
      const int r = next_region;
      next_region = (next_region + 1) % kRing;
      if (ev_pending[r]) {  // the kernel that read this region has finished
        hipError_t e = hipEventSynchronize(ev[r]);
        if (e != hipSuccess) return fail(MQA_ERR_HIP, "prefix cache: %s", hipGetErrorString(e));
        ev_pending[r] = false;
      }
      memcpy(arena + r * kRingBytes, pairs.data() + 2 * i0, (size_t)n * 16);
      const int64_t* cmd = reinterpret_cast<const int64_t*>(arena_dev + r * kRingBytes);
      hipLaunchKernelGGL(mqa::page_copy_kernel, dim3((n + 3) / 4), dim3(256), 0, stream, src, dst,
                         cmd, n, page_bytes);
      hipError_t e = hipGetLastError();
      if (e == hipSuccess) e = hipEventRecord(ev[r], stream);
      if (e != hipSuccess) return fail(MQA_ERR_HIP, "prefix cache copy: %s", hipGetErrorString(e));
      ev_pending[r] = true;
    }
    return MQA_OK;
  }
};

extern "C" {

int mqa_prefix_cache_create(void* host_arena, int64_t arena_bytes, int32_t num_slots,
                            const int32_t* slot_window, int32_t head_dim, int32_t flags,
                            mqa_prefix_cache** out) {
  if (!out) return fail(MQA_ERR_INVALID, "out is NULL");
  *out = nullptr;
  if (!host_arena) return fail(MQA_ERR_INVALID, "host_arena is NULL");
  if ((reinterpret_cast<uintptr_t>(host_arena) & 255) != 0)
    return fail(MQA_ERR_INVALID, "host_arena is not 256-byte aligned");
  if (num_slots < 1 || num_slots > 64) return fail(MQA_ERR_UNSUPPORTED, "num_slots %d not in [1, 64]", num_slots);
  if (head_dim != 64 && head_dim != 128) return fail(MQA_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (!slot_window) return fail(MQA_ERR_INVALID, "slot_window is NULL");
  for (int s = 0; s < num_slots; ++s)
    if (slot_window[s] < 0) return fail(MQA_ERR_INVALID, "slot_window[%d] < 0", s);
  if (flags != 0 && flags != MQA_PREFIX_HOST_ONLY) return fail(MQA_ERR_INVALID, "flags %d", flags);
  const int32_t pb = 32 * head_dim + 128;
  const int64_t entry = ((int64_t)pb + 255) & ~INT64_C(255);
  const int64_t base = kRing * kRingBytes;
  if (arena_bytes < base + entry)
    return fail(MQA_ERR_INVALID, "arena of %lld bytes holds no entry (%lld + %lld needed)",
                (long long)arena_bytes, (long long)base, (long long)entry);
  const int64_t cap = (arena_bytes - base) / entry;
  if (cap > INT32_MAX) return fail(MQA_ERR_UNSUPPORTED, "arena too large");
  uint8_t* dev = nullptr;
  if (flags != MQA_PREFIX_HOST_ONLY) {
    void* d = nullptr;
    hipError_t e = hipHostGetDevicePointer(&d, host_arena, 0);
    if (e != hipSuccess || !d)
      return fail(MQA_ERR_INVALID, "host_arena is not pinned host memory the GPU can address (%s)",
                  hipGetErrorString(e));
    dev = static_cast<uint8_t*>(d);
  }
  mqa_prefix_cache* c = new (std::nothrow) mqa_prefix_cache;
  if (!c) return fail(MQA_ERR_INVALID, "out of host memory");
  c->arena = static_cast<uint8_t*>(host_arena);
  c->arena_dev = dev;
  c->arena_bytes = arena_bytes;
  c->num_slots = num_slots;
  c->head_dim = head_dim;
  c->page_bytes = pb;
  c->entry_bytes = entry;
  c->entries_base = base;
  c->capacity = cap;
  c->window.assign(slot_window, slot_window + num_slots);
  // a node holds at least one entry, so there are never more nodes than entries
  c->nodes.resize((size_t)cap);
  c->slot_entry.assign((size_t)cap * num_slots, -1);
  c->free_nodes.reserve((size_t)cap);
  c->free_entries.reserve((size_t)cap);
  for (int64_t i = cap; i-- > 0;) {
    c->free_nodes.push_back((int32_t)i);
    c->free_entries.push_back((int32_t)i);
  }
  if (dev) {
    for (int r = 0; r < kRing; ++r) {
      hipError_t e = hipEventCreateWithFlags(&c->ev[r], hipEventDisableTiming);
      if (e != hipSuccess) {
        for (int q = 0; q < r; ++q) (void)hipEventDestroy(c->ev[q]);
        delete c;
        return fail(MQA_ERR_HIP, "prefix cache events: %s", hipGetErrorString(e));
      }
    }
  }
  *out = c;
  return ok();
}

int mqa_prefix_cache_destroy(mqa_prefix_cache* c) {
  if (!c) return ok();
  if (c->arena_dev) {
    for (int r = 0; r < kRing; ++r) {
      if (c->ev_pending[r]) (void)hipEventSynchronize(c->ev[r]);
      (void)hipEventDestroy(c->ev[r]);
    }
  }
  delete c;
  return ok();
}

int64_t mqa_prefix_cache_capacity(const mqa_prefix_cache* c) { return c ? c->capacity : -1; }

int64_t mqa_prefix_cache_entries(const mqa_prefix_cache* c) {
  return c ? c->capacity - (int64_t)c->free_entries.size() : -1;
}

int mqa_prefix_cache_stats(const mqa_prefix_cache* c, int64_t* out6) {
  if (!c || !out6) return fail(MQA_ERR_INVALID, "NULL argument");
  for (int i = 0; i < 6; ++i) out6[i] = c->stats[i];
  return ok();
}

int mqa_prefix_cache_lookup(mqa_prefix_cache* c, const int32_t* tokens, int64_t n,
                            int64_t* matched) {
  if (!c || !matched) return fail(MQA_ERR_INVALID, "NULL argument");
  if (n < 0 || (n > 0 && !tokens)) return fail(MQA_ERR_INVALID, "bad tokens");
  *matched = 0;
  ++c->stats[0];
  c->stats[1] += n;
  if (n < 2) return ok();
  // at least the last token is left to compute: it is the next query
  std::vector<int32_t> path;
  c->walk(tokens, (n - 1) / kPage, path);
  const int64_t P = c->restorable(path);
  c->touch_path(path, (size_t)P);
  *matched = P * kPage;
  c->stats[2] += *matched;
  return ok();
}

}  // extern "C"

namespace {

// Pages [0, n/16) of a sequence: the node path, created where missing.
// copy_slot(k, s, node) is called for every (page, slot) the entry must take.
template <typename F>
int insert_pages(mqa_prefix_cache* c, const int32_t* tokens, int64_t n, uint64_t (*avail)(void*, int64_t),
                 void* ctx, F copy_slot, int64_t* inserted) {
  const int64_t pages = n / kPage;
  ++c->epoch;
  std::vector<int32_t> path;
  uint64_t h = kHashSeed;
  int32_t parent = -1;
  int64_t added = 0;
  for (int64_t k = 0; k < pages; ++k) {
    const int32_t* t = tokens + k * kPage;
    h = chain_hash(h, t);
    const uint64_t have = avail(ctx, k);
    int32_t x = c->find(h, parent, t);
    if (x < 0) {
      if (!have) break;  // nothing of this page to keep: the path ends here
      // the new node's entries; every other entry is on this walk: the arena
      // is too small for more
      if (!c->reserve(__builtin_popcountll(have))) break;
      x = c->free_nodes.back();
      c->free_nodes.pop_back();
      Node& nd = c->nodes[x];
      nd.hash = h;
      nd.present = 0;
      nd.parent = parent;
      nd.children = 0;
      memcpy(nd.tokens, t, sizeof nd.tokens);
      nd.live = true;
      c->index.emplace(h, x);
      c->push_front(x);
      if (parent >= 0) ++c->nodes[parent].children;
    }
    Node& nd = c->nodes[x];
    nd.mark = c->epoch;
    const uint64_t missing = have & ~nd.present;
    if (missing && !c->reserve(__builtin_popcountll(missing))) break;
    for (int s = 0; s < c->num_slots; ++s)
      if (missing & (1ull << s)) {
        c->ent(x, s) = c->take_entry();
        copy_slot(k, s, c->ent(x, s));
        ++added;
      }
    nd.present |= missing;
    path.push_back(x);
    parent = x;
  }
  c->touch_path(path, path.size());
  c->stats[3] += added;
  if (inserted) *inserted = (int64_t)path.size();
  return MQA_OK;
}

struct TableView {
  const int32_t* table;
  int32_t batch, seq, max_pages, num_slots;
  int64_t num_pages;
  int32_t invalid;  // the table's mark for a page not held
  int32_t id(int s, int64_t k) const {
    return table[((int64_t)s * batch + seq) * max_pages + k];
  }
  bool valid(int s, int64_t k) const {
    if (k >= max_pages) return false;
    const int32_t p = id(s, k);
    return p != invalid && p >= 0 && p < num_pages;
  }
};

uint64_t table_avail(void* ctx, int64_t k) {
  const TableView* v = static_cast<const TableView*>(ctx);
  uint64_t m = 0;
  if (k >= v->max_pages) return 0;
  for (int s = 0; s < v->num_slots; ++s)
    if (v->valid(s, k)) m |= 1ull << s;
  return m;
}

struct HostPages {
  const uint64_t* present;
};

uint64_t host_avail(void* ctx, int64_t k) { return static_cast<HostPages*>(ctx)->present[k]; }

int check_seq_table(const mqa_prefix_cache* c, const int32_t* table, int32_t batch, int32_t seq,
                    int32_t max_pages) {
  if (!table) return fail(MQA_ERR_INVALID, "block_table_host is NULL");
  if (batch < 1 || seq < 0 || seq >= batch || max_pages < 1)
    return fail(MQA_ERR_INVALID, "bad batch/seq/max_pages (%d, %d, %d)", batch, seq, max_pages);
  (void)c;
  return MQA_OK;
}

}  // namespace

extern "C" {

int mqa_prefix_cache_insert(mqa_prefix_cache* c, const int32_t* tokens, int64_t n,
                            const mqa_kv_pool* pool, const int32_t* block_table_host,
                            int32_t batch, int32_t seq, int32_t max_pages, int32_t invalid_page,
                            void* stream, int64_t* cached_pages) {
  if (!c) return fail(MQA_ERR_INVALID, "prefix cache is NULL");
  if (!c->arena_dev) return fail(MQA_ERR_INVALID, "prefix cache was created host-only");
  if (n < 0 || (n > 0 && !tokens)) return fail(MQA_ERR_INVALID, "bad tokens");
  int rc = mqa::check_pool(pool);
  if (rc) return rc;
  if (pool->head_dim != c->head_dim) return fail(MQA_ERR_INVALID, "pool head_dim differs");
  rc = check_seq_table(c, block_table_host, batch, seq, max_pages);
  if (rc) return rc;
  TableView v{block_table_host, batch, seq, max_pages, c->num_slots, pool->num_pages,
              invalid_page};
  std::vector<int64_t> pairs;
  insert_pages(c, tokens, n, table_avail, &v,
               [&](int64_t k, int s, int32_t e) {
                 pairs.push_back((int64_t)v.id(s, k) * c->page_bytes);
                 pairs.push_back(c->entry_off(e));
               },
               cached_pages);
  if (!pairs.empty()) {
    rc = c->copy(static_cast<const uint8_t*>(pool->base), c->arena_dev, pairs,
                 static_cast<hipStream_t>(stream));
    if (rc) return rc;
  }
  return ok();
}

int mqa_prefix_cache_restore(mqa_prefix_cache* c, const int32_t* tokens, int64_t matched,
                             const mqa_kv_pool* pool, const int32_t* block_table_host,
                             int32_t batch, int32_t seq, int32_t max_pages, int32_t invalid_page,
                             void* stream) {
  if (!c) return fail(MQA_ERR_INVALID, "prefix cache is NULL");
  if (!c->arena_dev) return fail(MQA_ERR_INVALID, "prefix cache was created host-only");
  if (matched < 0 || matched % kPage || (matched > 0 && !tokens))
    return fail(MQA_ERR_INVALID, "matched %lld is not a multiple of 16", (long long)matched);
  int rc = mqa::check_pool(pool);
  if (rc) return rc;
  if (pool->head_dim != c->head_dim) return fail(MQA_ERR_INVALID, "pool head_dim differs");
  rc = check_seq_table(c, block_table_host, batch, seq, max_pages);
  if (rc) return rc;
  const int64_t P = matched / kPage;
  if (P > max_pages) return fail(MQA_ERR_INVALID, "matched beyond max_pages");
  std::vector<int32_t> path;
  c->walk(tokens, P, path);
  if ((int64_t)path.size() < P)
    return fail(MQA_ERR_INVALID, "only %lld of %lld pages are cached", (long long)path.size(),
                (long long)P);
  TableView v{block_table_host, batch, seq, max_pages, c->num_slots, pool->num_pages,
              invalid_page};
  std::vector<int64_t> pairs;
  for (int64_t k = 0; k < P; ++k)
    for (int s = 0; s < c->num_slots; ++s) {
      if (!v.valid(s, k)) continue;  // no page given: not needed by this step
      if (!(c->nodes[path[k]].present & (1ull << s)))
        return fail(MQA_ERR_INVALID, "page %lld of slot %d is not cached", (long long)k, s);
      pairs.push_back(c->entry_off(c->ent(path[k], s)));
      pairs.push_back((int64_t)v.id(s, k) * c->page_bytes);
    }
  if (!pairs.empty()) {
    rc = c->copy(c->arena_dev, static_cast<uint8_t*>(pool->base), pairs,
                 static_cast<hipStream_t>(stream));
    if (rc) return rc;
  }
  c->stats[5] += (int64_t)pairs.size() / 2;
  return ok();
}

int mqa_prefix_cache_insert_host(mqa_prefix_cache* c, const int32_t* tokens, int64_t n,
                                 const uint8_t* pages, const uint64_t* present,
                                 int64_t* cached_pages) {
  if (!c) return fail(MQA_ERR_INVALID, "prefix cache is NULL");
  if (n < 0 || (n > 0 && (!tokens || !pages || !present)))
    return fail(MQA_ERR_INVALID, "bad arguments");
  HostPages hp{present};
  const int64_t stride = (int64_t)c->num_slots * c->page_bytes;
  insert_pages(c, tokens, n, host_avail, &hp,
               [&](int64_t k, int s, int32_t e) {
                 memcpy(c->arena + c->entry_off(e), pages + k * stride + (int64_t)s * c->page_bytes,
                        (size_t)c->page_bytes);
               },
               cached_pages);
  return ok();
}

int mqa_prefix_cache_read_host(const mqa_prefix_cache* c, const int32_t* tokens, int64_t pages,
                               uint8_t* out, uint64_t* present) {
  if (!c) return fail(MQA_ERR_INVALID, "prefix cache is NULL");
  if (pages < 0 || (pages > 0 && (!tokens || !out || !present)))
    return fail(MQA_ERR_INVALID, "bad arguments");
  std::vector<int32_t> path;
  c->walk(tokens, pages, path);
  if ((int64_t)path.size() < pages)
    return fail(MQA_ERR_INVALID, "only %lld of %lld pages are cached", (long long)path.size(),
                (long long)pages);
  const int64_t stride = (int64_t)c->num_slots * c->page_bytes;
  for (int64_t k = 0; k < pages; ++k) {
    const int32_t x = path[k];
    for (int s = 0; s < c->num_slots; ++s) {
      uint8_t* o = out + k * stride + (int64_t)s * c->page_bytes;
      if (c->ent(x, s) >= 0)
        memcpy(o, c->arena + c->entry_off(c->ent(x, s)), (size_t)c->page_bytes);
      else
        memset(o, 0, (size_t)c->page_bytes);
    }
    present[k] = c->nodes[x].present;
  }
  return ok();
}

}  // extern "C"
