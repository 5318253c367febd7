/*
 * mqa_kv.h -- C ABI of the int8 multi-query KV-cache attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes is defined by these pages:
 *  - "Como funciona a inferência de IA, explicando claramente" (Red Hat),
 *    section "Por que o cache KV existe": a new token's query is compared with
 *    the key of every earlier token and the values are summed with those
 *    weights; K and V are computed once per token and kept in GPU memory.
 *    Section "Os modelos geram um token por vez": one new token per pass.
 *  - same page, section "O que os servidores de inferência em produção ...
 *    fazem a respeito?", item 1 (PagedAttention): the KV cache is cut into
 *    small fixed-size blocks placed anywhere, with a per-request table that
 *    says where each block is; item 3: prefix caching reuses cached K/V of a
 *    shared opening.
 *  - "Character.AI: inference optimization", section 03, technique table:
 *    multi-query attention in all layers (one K/V head), local attention with
 *    a horizon of 1024 interleaved with global layers (1 in 6 global), KV
 *    shared across layers; section 05: int8 quantisation of the attention KV
 *    cache; section 04: the KV of earlier turns is reused, so most turns
 *    append a new message to a cached prefix.
 *
 * Readings where the pages are silent: the softmax scale defaults to
 * 1/sqrt(head_dim); each token's K row and V row are coded as symmetric int8
 * with one fp32 scale each, scale = max|x| / 127 and code = rint(x / scale)
 * (ties to even) clamped to [-127, 127]; a window W covers the query's own
 * position and the W-1 before it (W = 0: the whole history); a context length
 * counts the current token (or appended chunk), whose K/V must already be
 * packed.  Pages hold 16 tokens.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless marked (host).
 *  - The caller owns every buffer (pool, tables, q, out, workspace).  The
 *    library never allocates or frees on these paths and keeps no pointer
 *    after it returns.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL
 *    for the null stream).  Buffers must stay alive until the stream passes
 *    the call.  Calls on one stream are ordered; concurrent calls on
 *    different streams must not share an output or workspace buffer.
 *  - Every entry point returns an mqa_status.  Host-visible arguments are all
 *    checked before anything is enqueued; on error nothing is enqueued or
 *    written and mqa_last_error() describes the problem.  A launch failure
 *    returns MQA_ERR_HIP.  Device-side contents (context lengths, page ids)
 *    are clamped in the kernels so that bad values cannot read or write out
 *    of bounds; they give undefined numbers instead.
 */
#ifndef MQA_KV_H
#define MQA_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MQA_KV_ABI_VERSION 5
#define MQA_PAGE_TOKENS 16
/* Largest max_context (tokens) that decode and append accept: 2^22 = 4,194,304.
 * It keeps the kernels' page and chunk arithmetic within 32 bits; a larger
 * bound is refused with MQA_ERR_UNSUPPORTED. */
#define MQA_MAX_CONTEXT (1 << 22)
/* Largest number of tokens one kv_pack_int8 call takes (of (token, KV head)
 * pairs for mqa_gqa_pack_bf16): 2^25, which keeps the launch within the
 * work-items one dispatch can hold.  Larger inputs are packed in several
 * calls; a larger count is refused with MQA_ERR_UNSUPPORTED. */
#define MQA_PACK_MAX_TOKENS (1 << 25)

typedef enum {
  MQA_OK = 0,
  MQA_ERR_INVALID = -1,      /* a bad argument                                  */
  MQA_ERR_UNSUPPORTED = -2,  /* a valid request this library does not implement */
  MQA_ERR_WORKSPACE = -3,    /* workspace missing or smaller than required      */
  MQA_ERR_HIP = -4           /* the HIP runtime reported an error               */
} mqa_status;

/* A dtype argument is an int on the wire; entry points reject values other
 * than these.  (C++ gives the enum int as its underlying type, so that an
 * out-of-range value passed in is still a valid value to test and reject.) */
#ifdef __cplusplus
typedef enum mqa_dtype : int {
#else
typedef enum mqa_dtype {
#endif
  MQA_F32 = 0,               /* IEEE binary32                                   */
  MQA_BF16 = 1               /* bfloat16 (upper half of a binary32)             */
} mqa_dtype;

/*
 * The paged int8 KV pool.  One KV head per slot (multi-query attention).
 * `base` points to `num_pages` page records of mqa_page_bytes(head_dim) bytes
 * each, 256-byte aligned.  A page holds 16 consecutive tokens of one slot of
 * one sequence: their int8 K codes, int8 V codes and fp32 K and V scales, all
 * in one record so that one page read brings everything attention needs.
 * Byte positions inside a record are given by mqa_page_offset(); the order is
 * chosen so that each GPU lane's matrix-core operand is one contiguous
 * 16-byte load.  A K or V code c (-127..127) is stored as the unsigned
 * byte c + 128 (c with its sign bit flipped), the form the fp16 operand
 * conversion takes as it is.  Pages of every slot come from the same pool;
 * which page holds which tokens is decided by the caller's block tables.
 */
typedef struct mqa_kv_pool {
  void*   base;
  int64_t num_pages;
  int32_t head_dim;          /* 64 or 128                                       */
  int32_t reserved;          /* must be 0                                       */
} mqa_kv_pool;

/* ABI version (MQA_KV_ABI_VERSION of the built library). */
int mqa_abi_version(void);

/* Text for the last non-OK status returned on this host thread ("" if none). */
const char* mqa_last_error(void);

/* Bytes of one page record: 32*head_dim + 128 (16 K rows, 16 V rows, 16+16
 * fp32 scales).  0 for an unsupported head_dim. */
size_t mqa_page_bytes(int32_t head_dim);

/*
 * Per-token KV bytes of a model, the formula of "Como funciona a inferência
 * de IA", section "Qual é o tamanho real do cache KV?":
 *   2 x num_layers x num_kv_heads x head_dim x dtype_bytes.
 * For this library's cache (one KV head, int8 codes) add 8 bytes of fp32
 * scales per token per slot.  Returns -1 for a negative argument.
 */
int64_t mqa_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads,
                               int32_t head_dim, int32_t dtype_bytes);

/*
 * Host-side layout query: byte offset inside a page record of token `token`
 * (0..15), channel `channel` (0..head_dim-1) of K (`which` = 0) or V (1), or
 * of that token's fp32 scale (`which` = 2 for K, 3 for V; `channel` ignored).
 * Writes the offset to *offset (host) and returns MQA_OK, or MQA_ERR_INVALID.
 */
int mqa_page_offset(int32_t head_dim, int32_t token, int32_t channel,
                    int32_t which, int64_t* offset);

/*
 * kv_pack_int8 -- quantise new tokens' K and V rows and write them into pages.
 *
 * Defined by: KV caching computes K and V once for each new token and keeps
 * them (Red Hat page, "Por que o cache KV existe"); the cache is int8
 * (Character.AI page, section 05) in fixed-size blocks found through a table
 * (Red Hat page, PagedAttention).
 *
 *  k, v          [num_tokens rows] of head_dim values of `src_dtype`; row t
 *                starts at element t*row_stride (row_stride >= head_dim).
 *                num_tokens is at most MQA_PACK_MAX_TOKENS per call.
 *  slot_mapping  int64 [num_tokens]: page*16 + offset_in_page of each token;
 *                a negative entry skips that token (padding).
 *  pool          (host) the page pool written.
 * For each token and each of K and V: a = max|x| over the row, s = a/127 in
 * fp32, code = clamp(rint(x/s), -127, 127) with an IEEE fp32 division (all
 * zeros when a = 0).  The result is bit-identical to that definition.
 * Entries pointing outside the pool are skipped.  Two tokens mapped to the
 * same position race; the caller must not do that.
 */
int kv_pack_int8(const void* k, const void* v, mqa_dtype src_dtype,
                 int64_t num_tokens, int64_t row_stride,
                 const int64_t* slot_mapping, const mqa_kv_pool* pool,
                 void* stream);

/*
 * Workspace for mqa_decode_attn / mqa_decode_step with the same shape
 * arguments and query dtype (the host arrays are read).  Contexts long enough
 * to be split across workgroups leave softmax partials (max, sum, weighted
 * values) there; the last of them to arrive merges them inside the same
 * kernel.  The first 8 MiB of a workspace hold the arrival counters (one per
 * wavefront of a workgroup, 8 or 4, per row block of a layer and sequence,
 * each on its own 128-byte line; at most 8192 such pairs per call), the
 * partials follow.  The size depends on the query dtype (fp32 queries are
 * carried as two fp16 terms, and a wavefront then takes 16 rows instead of
 * 32) and on the decode tuning in force (mqa_decode_tuning); query it again
 * after changing that.
 * Returns 0 when none is needed or the arguments are invalid (a following
 * call reports why).  The workspace must be zero-filled ONCE before its first
 * use (e.g. hipMemset after allocation); every call leaves the counters at
 * zero again, so later calls -- of any shape -- need no clearing.
 */
size_t mqa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                  int32_t num_layers, const int32_t* layer_slot,
                                  const int32_t* layer_window,
                                  int32_t max_context, int32_t head_dim,
                                  mqa_dtype q_dtype);

/*
 * Decode tuning (not part of what is computed: results depend on it only
 * through the rounding order of the merges).  Process-wide: a change applies
 * to every later call from any thread (each value is stored atomically; a call
 * racing with a change plans with the old or the new value of each), and a
 * workspace sized before a change may be too small after it.  Meant for tests
 * and tuning, not for a serving loop.  Each argument is 0 for "the planner
 * decides" or a forced value:
 *  waves       wavefronts per decode workgroup: 8 (one workgroup per CU) or
 *              4 (two per CU).  The planner takes 4 only when the 8-wavefront
 *              plan leaves more than 15 % of the CUs idle while splitting
 *              every item into at least 2 chunks, and 4 fills at least 10 %
 *              more of the slots with at most 8 chunks per item.
 *  rows        query rows per row block: 8, 16 or 32 (at most 16 with fp32
 *              queries).
 *  target_wgs  workgroups of 8 wavefronts the planner aims for (default 256,
 *              one per CU of an MI355X).
 * Starts from the environment variables MQA_DECODE_WAVES, MQA_DECODE_ROWS and
 * MQA_DECODE_TARGET_WGS.  Returns MQA_OK, or MQA_ERR_INVALID (nothing
 * changed) for a value outside those sets or a negative target.
 */
int mqa_decode_tuning(int32_t waves, int32_t rows, int32_t target_wgs);

/*
 * mqa_decode_attn -- one decode step of multi-query attention over the paged
 * int8 cache: every query head of every listed layer of every sequence.
 *
 * Defined by: one new token per pass, whose query is compared with every
 * cached key and whose output is the weighted sum of cached values (Red Hat
 * page, "Os modelos geram um token por vez" and "Por que o cache KV existe");
 * one shared K/V head per layer, local layers with a horizon, KV shared across
 * layers (Character.AI page, section 03 table).
 *
 *  q             [num_layers][batch][num_q_heads][head_dim] of `q_dtype`.
 *  out           fp32, same shape.  out = softmax(scale * q.khat^T) vhat over
 *                the attended keys, khat = sK*codeK, vhat = sV*codeV.
 *  block_table   int32 [num_slots][batch][max_pages_per_seq]: page ids in
 *                the pool of the logical pages 0,1,2,... of each sequence in
 *                each slot.  Entries up to page ceil(max_context/16)-1 of a
 *                row may be read even where the sequence does not attend them
 *                (the page ids are fetched for the bound's range before the
 *                length is known), but no page is ever loaded through such an
 *                entry: they may hold any value.
 *  context_lens  int32 [batch]: cached tokens of each sequence including the
 *                current one (which sits at position context_len-1).  Must
 *                lie in [1, max_context]; a length <= 0 gives zeros.
 *  max_context   (host) upper bound of context_lens, used to plan the launch
 *                without reading device memory; at most MQA_MAX_CONTEXT.
 *  layer_slot    (host) int32 [num_layers]: the KV slot each layer reads.
 *                Layers that read the same slot with the same window are
 *                served from one KV read (cross-layer KV sharing).
 *  layer_window  (host) int32 [num_layers]: 0 = global, W > 0 = the last W
 *                positions (the query's own included).
 *  softmax_scale <= 0 selects 1/sqrt(head_dim); NaN, an infinity or a scale
 *                whose product with log2(e) overflows fp32 is refused.
 *  workspace     at least mqa_decode_workspace_bytes(...) bytes, 256-byte
 *                aligned, zero-filled before its first use (see above).  May
 *                be NULL when that size is 0.  Calls sharing one workspace
 *                must not overlap (calls on one stream never do).
 * Supported: head_dim 64 or 128; q_dtype MQA_F32 or MQA_BF16; out fp32.
 */
int mqa_decode_attn(const void* q, mqa_dtype q_dtype, float* out,
                    const mqa_kv_pool* pool, const int32_t* block_table,
                    int32_t max_pages_per_seq, const int32_t* context_lens,
                    int32_t max_context, int32_t batch, int32_t num_q_heads,
                    int32_t num_layers, int32_t num_slots,
                    const int32_t* layer_slot, const int32_t* layer_window,
                    float softmax_scale, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * mqa_decode_step -- kv_pack_int8 of the current token fused into
 * mqa_decode_attn: one launch stores every slot's new K/V row and runs the
 * decode attention that reads it.
 *
 * Defined by: a new token's K and V are computed once and kept in the cache
 * (Red Hat page, "Por que o cache KV existe"), as int8 (Character.AI page,
 * section 05); its query then attends the cache including itself (same
 * sections as mqa_decode_attn).
 *
 *  k_new, v_new  [num_slots][batch][head_dim] of `kv_dtype` (MQA_F32 or
 *                MQA_BF16): the current token's K and V row of each slot.
 * For every slot that some layer reads and every sequence b with
 * context_lens[b] >= 1, the rows of (slot, b) are coded exactly as
 * kv_pack_int8 codes them and stored at position context_lens[b] - 1, i.e.
 * page block_table[slot][b][(ctx-1)/16], token (ctx-1)%16 -- the same bytes
 * kv_pack_int8 followed by mqa_decode_attn would leave -- and `out` equals
 * what that pair of calls returns.  Rows of slots no layer reads are not
 * stored.  The page holding the current token must not be shared with
 * another sequence in the same call.  Other arguments, the workspace and the
 * error behaviour are those of mqa_decode_attn.
 */
int mqa_decode_step(const void* q, mqa_dtype q_dtype, float* out,
                    const void* k_new, const void* v_new, mqa_dtype kv_dtype,
                    const mqa_kv_pool* pool, const int32_t* block_table,
                    int32_t max_pages_per_seq, const int32_t* context_lens,
                    int32_t max_context, int32_t batch, int32_t num_q_heads,
                    int32_t num_layers, int32_t num_slots,
                    const int32_t* layer_slot, const int32_t* layer_window,
                    float softmax_scale, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * mqa_append_attn -- causal attention of a multi-token chunk appended to a
 * cached prefix (a new turn after a cross-turn cache hit, or prefill on top of
 * a reused prefix).
 *
 * Defined by: the KV of earlier turns is kept and reused, so a new message is
 * processed on top of the cached prefix (Character.AI page, section 04;
 * Red Hat page, prefix caching); each token attends every earlier token and
 * itself (Red Hat page, "Por que o cache KV existe"), limited by the layer's
 * window (Character.AI page, section 03 table).
 *
 *  q             [num_layers][total_q][num_q_heads][head_dim] of `q_dtype`;
 *                sequence b owns rows cu_q_lens[b] .. cu_q_lens[b+1]-1.
 *  out           fp32, same shape.
 *  context_lens  int32 [batch]: cached tokens including the whole chunk,
 *                whose K/V must already be packed.  Token t of sequence b sits
 *                at position context_lens[b] - q_len_b + t.
 *  cu_q_lens     int32 [batch+1]: prefix sums of the chunk lengths
 *                (cu_q_lens[0] = 0, cu_q_lens[batch] = total_q).
 *  max_q_len     (host) upper bound of the chunk lengths.
 * Device-side lengths that break these rules are not errors the host can
 * see: rows of a chunk past max_q_len, and every row of a sequence whose rows
 * fall outside [0, total_q), are left unwritten; nothing is read or written
 * out of bounds.
 * Other arguments as for mqa_decode_attn.  No workspace is needed.
 */
int mqa_append_attn(const void* q, mqa_dtype q_dtype, float* out,
                    const mqa_kv_pool* pool, const int32_t* block_table,
                    int32_t max_pages_per_seq, const int32_t* context_lens,
                    const int32_t* cu_q_lens, int32_t max_context,
                    int32_t max_q_len, int32_t total_q, int32_t batch,
                    int32_t num_q_heads, int32_t num_layers, int32_t num_slots,
                    const int32_t* layer_slot, const int32_t* layer_window,
                    float softmax_scale, void* stream);

/* ---------------------------------------------------------------------------
 * Host-side memory management of the paged cache.  Nothing below launches
 * work or touches device memory; every pointer is a HOST pointer.
 * ------------------------------------------------------------------------- */

/*
 * Bytes of KV cache one sequence holds at `context` tokens (its positions
 * 0 .. context-1), for a model whose layer l reads slot layer_slot[l] through
 * window layer_window[l] (0 = global).  The techniques of "Character.AI:
 * inference optimization", section 03, technique table, each show up here:
 *  - multi-query attention: num_kv_heads = 1 (grouped-query: 8);
 *  - KV shared across layers: each distinct slot is stored once;
 *  - hybrid local/global attention: a slot that only windowed layers read
 *    keeps only the tokens its widest window still reaches,
 *    max(0, context - W) .. context-1 (see mqa_page_table_advance);
 * and section 05 (int8 KV cache) through code_bytes = 1 and scale_bytes = 4
 * (one fp32 scale per token, KV head and K or V); bf16: 2 and 0.
 * Per token and slot: 2 x num_kv_heads x (head_dim x code_bytes +
 * scale_bytes), which with one slot per layer and no scales is the formula of
 * "Como funciona a inferência de IA", section "Qual é o tamanho real do cache
 * KV?".  page_tokens > 0 counts whole pages of that many tokens (what a paged
 * pool holds: MQA_PAGE_TOKENS for this library); 0 counts tokens exactly.
 * Returns -1 for a negative argument or a NULL map with num_layers > 0.
 */
int64_t mqa_kv_footprint_bytes(int32_t num_layers, const int32_t* layer_slot,
                               const int32_t* layer_window, int32_t num_kv_heads,
                               int32_t head_dim, int32_t code_bytes, int32_t scale_bytes,
                               int64_t context, int32_t page_tokens);

/*
 * Page table with recycling of windowed slots: a host object that hands out
 * the pool pages first_page .. first_page+num_pages-1 to (slot, sequence)
 * pairs as sequences grow, and takes back every page of a windowed slot once
 * no later step can read it (all its tokens lie before the window of the
 * sequence's earliest remaining query).  Pages are fixed-size blocks placed
 * anywhere, found through a per-request table ("Como funciona a inferência
 * de IA", section "O que os servidores ... fazem a respeito?", item 1); the
 * local layers' horizon ("Character.AI: inference optimization", section 03)
 * bounds what a local slot must keep to ceil(W/16) + 1 pages for decode
 * steps.  The object writes the rows of the caller's host block table
 * ([num_slots][batch][max_pages] int32, the layout mqa_decode_attn reads once
 * copied to the device); entries of pages not held are `invalid_page` (a
 * value outside the managed range: -1, or a poison page of the caller's).
 * Not thread-safe: one object per host thread or external locking.
 *
 * create:   slot_window[num_slots] (0 = global).  *out receives the object;
 *           destroy frees it.
 * advance:  sequence `seq` now holds `context` tokens, the last `new_tokens`
 *           of which form this step's queries (1 for a decode step, the
 *           chunk length for mqa_append_attn).  Frees the pages of windowed
 *           slots that fall entirely before max(0, context - new_tokens + 1 -
 *           W), then gives the sequence pages up to token context-1 in every
 *           slot.  The sequence's first call writes its whole row of each
 *           slot in block_table; later calls write only the entries they
 *           change (block_table may be NULL to keep no mirror).  Errors
 *           (nothing changes): context below the sequence's, beyond
 *           max_pages x 16, new_tokens outside [1, context], an earliest
 *           query before the last step's (MQA_ERR_INVALID); the free list
 *           too short (MQA_ERR_UNSUPPORTED).
 * advance_all: one step of the whole batch in one call: context[batch] and
 *           new_tokens[batch] (host) as for advance, new_tokens[b] = 0 for a
 *           sequence that does not step.  All or nothing: on any error no
 *           sequence changes.  Every stepping sequence frees before any grows.
 * release:  the sequence ends: all its pages go back; its rows become
 *           invalid_page.
 * free_pages / held_pages: free-list length; pages (seq, slot) holds (-1 on
 *           a bad argument).
 * slot_mapping: page*16 + offset of tokens start .. start+count-1 of (seq,
 *           slot), the form kv_pack_int8 takes; MQA_ERR_INVALID if one of
 *           them has no page.
 */
typedef struct mqa_page_table mqa_page_table;
int mqa_page_table_create(int32_t first_page, int32_t num_pages, int32_t num_slots,
                          const int32_t* slot_window, int32_t batch, int32_t max_pages,
                          int32_t invalid_page, mqa_page_table** out);
int mqa_page_table_destroy(mqa_page_table* table);
int mqa_page_table_advance(mqa_page_table* table, int32_t seq, int64_t context,
                           int32_t new_tokens, int32_t* block_table);
int mqa_page_table_advance_all(mqa_page_table* table, const int64_t* context,
                               const int32_t* new_tokens, int32_t* block_table);
int mqa_page_table_release(mqa_page_table* table, int32_t seq, int32_t* block_table);
int64_t mqa_page_table_free_pages(const mqa_page_table* table);
int64_t mqa_page_table_held_pages(const mqa_page_table* table, int32_t seq, int32_t slot);
int mqa_page_table_slot_mapping(const mqa_page_table* table, int32_t seq, int32_t slot,
                                int64_t start, int32_t count, int64_t* out);

/*
 * Cross-turn prefix cache ("Character.AI: inference optimization", section
 * 04: the KV of earlier turns is kept in host memory in a tree-structured LRU
 * cache indexed by a rolling hash of every prefix, and a new turn reuses the
 * longest cached prefix; "Como funciona a inferência de IA", section "O que
 * os servidores ... fazem a respeito?", item 3: prefix caching).
 *
 * A node of the tree is one page (16 tokens) of one prefix, so the tree is a
 * radix tree over pages; it owns one arena entry per KV slot whose page it
 * holds, byte for byte as in the pool (a windowed slot's early pages are
 * usually recycled before a turn is offloaded, so most nodes of a long
 * dialogue hold only the global slots).  A node is found by a 64-bit hash
 * chained page by page over the token ids and confirmed by its parent and
 * its 16 tokens, so a hash collision can never return another prefix.
 * Eviction removes the least recently used leaf, so a cached page's prefix
 * is always cached.
 *
 * Memory: `host_arena` is pinned host memory the caller owns (hipHostMalloc,
 * or a pinned torch tensor), 256-byte aligned, kept alive until destroy.  The
 * first 256 KiB hold a command ring (the copy lists the kernels read); the
 * rest is cut into entries of mqa_page_bytes(head_dim) bytes (rounded up to
 * 256), one per cached (page, slot): mqa_prefix_cache_capacity() of them,
 * mqa_prefix_cache_entries() in use.  The object's own bookkeeping is host
 * memory it allocates at create.
 *
 * Copies run as one kernel per 4096 pages (one wavefront per page, over the
 * host link) enqueued on `stream`.  Calls are not thread-safe; use one
 * stream per cache, or order the streams: an insert may evict and refill an
 * entry that an earlier restore reads.
 *
 * create:  slot_window[num_slots] as for mqa_page_table_create (num_slots
 *          <= 64).  flags = MQA_PREFIX_HOST_ONLY: no GPU is used (host
 *          inserts and reads only; for tests and host-side loading).
 * lookup:  the longest cached prefix of tokens[0..n) that a step whose
 *          earliest query is the token right after it can use: a multiple of
 *          16, at most n-1 (the last token is always left to compute as the
 *          next query), such that every page a global slot reads and every
 *          page of a windowed slot within its window is cached.  Marks the
 *          pages used.  *matched receives the token count (host).
 * restore: for pages k < matched/16 of sequence `seq` and every slot whose
 *          entry block_table_host[slot][seq][k] is a pool page (in range and
 *          not `invalid_page`, the table's mark for a page not held), copies
 *          the cached page into it (host -> device).  block_table_host is the
 *          host mirror of the step's block table ([num_slots][batch]
 *          [max_pages]); with mqa_page_table_advance(seq, n, n - matched) it
 *          gives exactly the pages the step reads.  MQA_ERR_INVALID (nothing
 *          enqueued) if a needed page is not cached.
 * insert:  the full pages of tokens[0..n) of sequence `seq`, from the pool
 *          pages its table rows give (entries equal to `invalid_page` or out
 *          of range: not held) (device -> host), for every page and
 *          slot not yet cached; creates nodes as needed, evicting least
 *          recently used leaves.  Stops early (still MQA_OK) when the arena
 *          cannot take more or a page has no slot at all; *cached_pages
 *          (host, may be NULL) receives how many leading pages are cached
 *          afterwards.
 * insert_host / read_host: the same with page bytes in host memory laid out
 *          [page][slot][mqa_page_bytes] and a slot mask per page (present).
 * stats:   out6 = lookups, tokens asked, tokens matched, entries inserted,
 *          entries evicted, entries restored (an entry: one page of one slot).
 */
/*
 * Grouped-query bf16 decode: the baseline of "Character.AI: inference
 * optimization", section 03, technique table (multi-query attention cuts the
 * KV cache 8X against grouped-query attention), on the same harness, so the
 * factor can be measured as bytes and time.  One layer; num_kv_heads K/V
 * heads in bf16, query head j reading KV head j / (num_q_heads /
 * num_kv_heads) (at most 16 query heads per KV head).
 *
 * Pool: num_pages records of mqa_gqa_page_bytes() bytes (256-byte aligned),
 * one per 16 tokens of one sequence, holding every KV head: for head h,
 * 64*head_dim bytes at h*64*head_dim, its 16 tokens' K then V in bf16
 * matrix-core operand order (the order mqa_gqa_pack_bf16 writes).
 *
 * pack:    k, v (device) bf16 [num_tokens][num_kv_heads][head_dim], with
 *          num_tokens*num_kv_heads at most MQA_PACK_MAX_TOKENS per call;
 *          slot_mapping int64 [num_tokens] = page*16 + position in page
 *          (negative or past the pool: skipped).
 * decode:  q bf16 [batch][num_q_heads][head_dim]; out fp32 same shape;
 *          block_table int32 [batch][max_pages]; context_lens int32 [batch]
 *          (the query at context-1); max_context at most MQA_MAX_CONTEXT;
 *          window 0 = global.  Contexts split over
 *          workgroups use `workspace` (mqa_gqa_decode_workspace_bytes(),
 *          no clearing needed) and a second small kernel merges them.
 * Errors as for the other entry points.
 */
size_t mqa_gqa_page_bytes(int32_t num_kv_heads, int32_t head_dim);
int mqa_gqa_pack_bf16(const void* k, const void* v, int64_t num_tokens,
                      const int64_t* slot_mapping, void* pool, int64_t num_pages,
                      int32_t num_kv_heads, int32_t head_dim, void* stream);
size_t mqa_gqa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t max_context, int32_t window, int32_t head_dim);
int mqa_gqa_decode_bf16(const void* q, float* out, const void* pool, int64_t num_pages,
                        int32_t num_kv_heads, int32_t head_dim, const int32_t* block_table,
                        int32_t max_pages, const int32_t* context_lens, int32_t max_context,
                        int32_t batch, int32_t num_q_heads, int32_t window, float softmax_scale,
                        void* workspace, size_t workspace_bytes, void* stream);

#define MQA_PREFIX_HOST_ONLY 1
typedef struct mqa_prefix_cache mqa_prefix_cache;
int mqa_prefix_cache_create(void* host_arena, int64_t arena_bytes, int32_t num_slots,
                            const int32_t* slot_window, int32_t head_dim, int32_t flags,
                            mqa_prefix_cache** out);
int mqa_prefix_cache_destroy(mqa_prefix_cache* cache);
int64_t mqa_prefix_cache_capacity(const mqa_prefix_cache* cache);
int64_t mqa_prefix_cache_entries(const mqa_prefix_cache* cache);
int mqa_prefix_cache_stats(const mqa_prefix_cache* cache, int64_t* out6);
int mqa_prefix_cache_lookup(mqa_prefix_cache* cache, const int32_t* tokens, int64_t n,
                            int64_t* matched);
int mqa_prefix_cache_restore(mqa_prefix_cache* cache, const int32_t* tokens, int64_t matched,
                             const mqa_kv_pool* pool, const int32_t* block_table_host,
                             int32_t batch, int32_t seq, int32_t max_pages, int32_t invalid_page,
                             void* stream);
int mqa_prefix_cache_insert(mqa_prefix_cache* cache, const int32_t* tokens, int64_t n,
                            const mqa_kv_pool* pool, const int32_t* block_table_host,
                            int32_t batch, int32_t seq, int32_t max_pages, int32_t invalid_page,
                            void* stream, int64_t* cached_pages);
int mqa_prefix_cache_insert_host(mqa_prefix_cache* cache, const int32_t* tokens, int64_t n,
                                 const uint8_t* pages, const uint64_t* present,
                                 int64_t* cached_pages);
int mqa_prefix_cache_read_host(const mqa_prefix_cache* cache, const int32_t* tokens,
                               int64_t pages, uint8_t* out, uint64_t* present);

/*
 * mqa_decode_step_noalloc -- mqa_decode_step for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same computation, outputs and
 * stored bytes as mqa_decode_step, with no workspace argument.  Its scratch
 * (arrival counters and partial softmax records) is a static device array of
 * the library of MQA_DECODE_STATIC_SCRATCH_BYTES, one copy per GPU, held
 * until the process ends; the call allocates nothing and calls no
 * hipMalloc/hipFree.  The first call on a device looks up that device's copy
 * (with the device current) and clears its counters with a small kernel on
 * `stream`.  Every call on one GPU shares that GPU's copy, which keeps the
 * last call's contents: calls that overlap on one GPU (other streams,
 * other host threads) race and give undefined results; calls on one stream
 * never overlap.  A launch whose plan needs more scratch than the array
 * holds (mqa_decode_workspace_bytes of the same arguments, fp32 or bf16 q)
 * returns MQA_ERR_WORKSPACE before anything is enqueued.  Other arguments
 * and errors: those of mqa_decode_step.
 */
#define MQA_DECODE_STATIC_SCRATCH_BYTES (40u << 20)
int mqa_decode_step_noalloc(const void* q, mqa_dtype q_dtype, float* out,
                            const void* k_new, const void* v_new, mqa_dtype kv_dtype,
                            const mqa_kv_pool* pool, const int32_t* block_table,
                            int32_t max_pages_per_seq, const int32_t* context_lens,
                            int32_t max_context, int32_t batch, int32_t num_q_heads,
                            int32_t num_layers, int32_t num_slots,
                            const int32_t* layer_slot, const int32_t* layer_window,
                            float softmax_scale, void* stream);

/*
 * mqa_hbm_read_probe -- a streaming read of device memory, to measure the
 * bandwidth a plain read reaches on this GPU (decode attention streams KV
 * bytes, whose volume sets its cost: Character.AI page, section 02).  Not
 * part of the method.
 *
 *  src         device buffer of `bytes` bytes (a positive multiple of 16,
 *              16-byte aligned), read once with 128-bit loads.
 *  sink        device uint32 [sink_words], sink_words >= MQA_PROBE_SINK_WORDS.
 *              Word g (g < MQA_PROBE_SINK_WORDS) receives the XOR of the
 *              32-bit words of the g-th of MQA_PROBE_SINK_WORDS equal
 *              contiguous ranges of src (0 for an empty range), so the XOR of
 *              all sink words equals the XOR of all 32-bit words of src.
 * Asynchronous on `stream`.  Returns MQA_OK or MQA_ERR_INVALID / MQA_ERR_HIP.
 */
#define MQA_PROBE_SINK_WORDS 4096
int mqa_hbm_read_probe(const void* src, int64_t bytes, uint32_t* sink, int32_t sink_words,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MQA_KV_H */
