/*
 * pagedkv.h -- C ABI of a paged KV-cache decode-attention library for AMD
 * MI355X (gfx950).
 *
 * What the library implements, from the pages it follows:
 *
 *  - Page "生成一个字，为什么要背一整本账", section
 *    "PagedAttention：把操作系统的老智慧搬进推理引擎": each sequence's KV cache
 *    is cut into fixed-size blocks (16 tokens by default) that may sit anywhere
 *    in device memory, mapped by a per-sequence block table; blocks are taken
 *    on demand; shared prefixes are stored once, reference counted and copied
 *    on write where sequences diverge.
 *  - Page "AI 陪读顶会论文（三）：KV Cache 显存占用计算与 PagedAttention 原理拆解",
 *    section "为什么自回归解码…必须使用 KV Cache": at each decode step only the
 *    new token's k and v are appended, and its query attends with
 *    softmax(q K^T / sqrt(d)) V over every cached token, itself included;
 *    section "PagedAttention 的破局哲学": the logical-to-physical block figure
 *    and the three innovations (non-contiguous blocks, on-demand allocation,
 *    copy-on-write for branches).
 *  - Page "生成一个字…", section "显存账本": grouped-query attention, several
 *    query heads sharing one KV head; section "再往后：压 KV 的三条路线": FP8
 *    K/V with per-channel scales, and a sliding attention window.
 *
 * Conventions for every call
 *  - Return value: PKV_OK (0) or a negative pkv_status.  On failure
 *    pkv_last_error() returns a message for the calling thread.  No C++
 *    exception crosses this interface.
 *  - Host calls (block tables) validate every argument first and change no
 *    state when they fail (strong guarantee).
 *  - Device calls are asynchronous on the given stream (a hipStream_t; NULL is
 *    the default stream).  They validate their arguments on the host and
 *    return PKV_E_HIP if the launch itself fails; errors during execution
 *    surface at the caller's next synchronisation.
 *  - The pool object owns host metadata only (tables, lengths, reference
 *    counts, the free-block queue).  Every device pointer is borrowed: the
 *    caller allocates it, keeps it alive while the pool uses it and frees it.
 *  - No internal locking: calls on one pool must be serialised by the caller.
 *    Device work on one pool must be ordered on one stream:
 *    kv_pool_copy_blocks, then paged_kv_append, then paged_attention_decode.
 *
 * Device memory layout of one pool (both buffers contiguous, caller-owned):
 *    x = 16 / bytes_per_element   (4 for fp32, 8 for fp16/bf16, 16 for fp8)
 *    v = min(block_size, t), t = 16 for fp32, 32 for fp16/bf16, 64 for fp8
 *    K: [num_layers][num_blocks][num_kv_heads][head_dim / x][block_size][x]
 *    V: [num_layers][num_blocks][num_kv_heads][block_size / v][head_dim][v]
 *  Token `slot` of a block-table lives in physical block slot / block_size at
 *  offset slot % block_size.  Each (block, KV head) tile of K and of V is one
 *  contiguous run of block_size * head_dim elements.  K keeps 16-byte groups
 *  of channels of consecutive tokens together; V is stored channel-major in
 *  runs of v tokens (the tokens the decode reads at a time), which is plain
 *  channel-major [head_dim][block_size] when block_size <= t.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pkv_status;
enum {
  PKV_OK = 0,
  PKV_E_INVAL = -1,        /* bad argument, unknown sequence, bad state */
  PKV_E_OOM = -2,          /* not enough free blocks; nothing was changed */
  PKV_E_DTYPE = -3,        /* dtype combination not supported */
  PKV_E_UNSUPPORTED = -4,  /* shape without a kernel (head_dim, block size, group) */
  PKV_E_HIP = -5,          /* a HIP runtime call failed */
  PKV_E_INTERNAL = -6      /* unexpected failure (e.g. host allocation) */
};

/* Element types.  Stored as int32_t in the structs below. */
enum {
  PKV_F32 = 0,
  PKV_F16 = 1,
  PKV_BF16 = 2,
  PKV_FP8_E4M3 = 3   /* OCP E4M3: bias 7, max finite 448, NaN = S.1111.111 */
};

typedef void* pkv_stream;           /* a hipStream_t */
typedef struct kv_pool kv_pool;     /* opaque */

/* One whole-block copy (copy-on-write): physical block src -> dst. */
typedef struct {
  int32_t src;
  int32_t dst;
} kv_block_copy;

typedef struct {
  int32_t num_layers;     /* >= 1 */
  int32_t num_kv_heads;   /* >= 1 */
  int32_t head_dim;       /* device kernels: 64 or 128 */
  int32_t block_size;     /* tokens per block; device kernels: 16, 32, 64, 128 */
  int32_t num_blocks;     /* physical blocks per layer, >= 1 */
  int32_t kv_dtype;       /* PKV_F32 / PKV_F16 / PKV_BF16 / PKV_FP8_E4M3 */
  void* k_cache;          /* device, layout above; may be NULL for a host-only pool */
  void* v_cache;          /* device, layout above; may be NULL for a host-only pool */
  /* FP8 only (NULL otherwise): device fp32 [num_layers][num_kv_heads][head_dim],
   * i.e. each array holds num_layers * num_kv_heads * head_dim floats (the
   * kernels index it so; a shorter buffer is read past its end).  Per-channel
   * scales (page "生成一个字…", section "再往后：压 KV 的三条路线"): a stored code c
   * stands for e4m3(c) * scale; appends encode x * inv_scale, where inv_scale
   * is the caller's fp32 value of 1/scale. */
  const float* k_scale;
  const float* v_scale;
  const float* k_inv_scale;
  const float* v_inv_scale;
  /* Host, optional: initial order of the free-block queue, a permutation of
   * 0..num_blocks-1 (NULL: ascending).  Copied at creation. */
  const int32_t* free_order;
} kv_pool_desc;

/* Bytes one of the two device buffers (K or V) of a pool must hold:
 * num_layers * num_blocks * num_kv_heads * block_size * head_dim * element size
 * -- half the byte formula of page "生成一个字…" (opening section: 2 x layers x
 * KV heads x head_dim x tokens x bytes) at num_blocks * block_size tokens. */
pkv_status kv_pool_cache_bytes(const kv_pool_desc* desc, size_t* bytes_out);

/* Create the host side of a pool: the physical block pool of page "生成一个字…",
 * section "PagedAttention：…" (fixed-size blocks anywhere in device memory,
 * handed out on demand).  Validates the descriptor (positive sizes, a
 * permutation in free_order, scales present iff FP8).  All blocks start free
 * with reference count 0, queued in free_order.  *out receives the handle;
 * on failure *out is set to NULL and nothing stays allocated. */
pkv_status kv_pool_create(const kv_pool_desc* desc, kv_pool** out);
/* Release the host side.  Device buffers are not touched.  NULL is a no-op. */
void kv_pool_destroy(kv_pool* pool);

/* Number of free physical blocks (same section: blocks are taken on demand,
 * so this is what the pool can still give out).  PKV_E_INVAL on NULL. */
pkv_status kv_pool_num_free(const kv_pool* pool, int32_t* out);
/* Reference count of a physical block (0 = free): how many sequences hold it
 * (same section: a shared prefix is stored once and counted; page
 * "AI 陪读顶会论文（三）", section "PagedAttention 的破局哲学", innovation 3).
 * PKV_E_INVAL for a block outside 0..num_blocks-1. */
pkv_status kv_pool_refcount(const kv_pool* pool, int32_t block, int32_t* out);
/* The free-block queue, front first (the pages leave the free-block policy
 * open; this library hands out the front and queues freed blocks at the
 * back): up to cap ids into out (host), the queue length into *n_out. */
pkv_status kv_pool_free_list(const kv_pool* pool, int32_t* out, int32_t cap, int32_t* n_out);

/* ---- block tables (host only; page "生成一个字…", section "PagedAttention：…";
 *      page "AI 陪读顶会论文（三）", section "PagedAttention 的破局哲学") ---- */

/* New empty sequence (length 0, no blocks).  Ids count up from 0 and are
 * never reused. */
pkv_status block_table_alloc(kv_pool* pool, int32_t* seq_out);

/* Reserve slots for n_tokens new tokens of seq (token n of a sequence, counted
 * from 0, goes to slot table[n / block_size] * block_size + n % block_size).
 *  - A block is taken from the front of the free queue exactly when a token
 *    with n % block_size == 0 arrives (on-demand allocation).
 *  - If the first new token falls into a partly filled last block whose
 *    reference count is > 1, that block is copied on write: a fresh block is
 *    taken, {old, new} is written to cow_out[0], the old block's count drops
 *    by one and the table points at the new block.  The caller must run
 *    kv_pool_copy_blocks on the pairs before appending tokens.
 * slots_out: host int64 [n_tokens]; cow_out: host, capacity >= 1;
 * *n_cow_out: 0 or 1.  PKV_E_OOM (state unchanged) if the free queue cannot
 * supply every block the call needs. */
pkv_status block_table_append(kv_pool* pool, int32_t seq, int32_t n_tokens,
                              int64_t* slots_out, kv_block_copy* cow_out,
                              int32_t* n_cow_out);

/* One new token for each of n distinct sequences, processed in the given
 * order, all or nothing.  slots_out: host int64 [n]; cow_out: host, capacity
 * >= n; *n_cow_out receives the number of copies (in processing order). */
pkv_status block_table_append_batch(kv_pool* pool, const int32_t* seqs, int32_t n,
                                    int64_t* slots_out, kv_block_copy* cow_out,
                                    int32_t* n_cow_out);

/* New sequence sharing every block of parent (each block's count + 1). */
pkv_status block_table_fork(kv_pool* pool, int32_t parent, int32_t* child_out);

/* Drop a sequence: each block's count - 1, in table order; a block reaching 0
 * goes to the back of the free queue.  The id becomes invalid. */
pkv_status block_table_free(kv_pool* pool, int32_t seq);

/* n forks at once: children_out[i] receives a new sequence sharing every
 * block of parents[i] (a parent may appear several times).  Children get
 * consecutive ids in order.  All or nothing: an unknown parent changes
 * nothing.  children_out: host int32 [n]. */
pkv_status block_table_fork_batch(kv_pool* pool, const int32_t* parents, int32_t n,
                                  int32_t* children_out);

/* n frees at once, in the given order, each as block_table_free.  All or
 * nothing: an unknown or repeated id changes nothing. */
pkv_status block_table_free_batch(kv_pool* pool, const int32_t* seqs, int32_t n);

/* Sliding-window release (page "生成一个字…", section "再往后：压 KV 的三条路线":
 * with a window only the last stretch of tokens is attended, so the cache a
 * sequence holds can stay bounded by the window): every block of seq whose
 * tokens all lie before `token` is handed back -- its count drops by one, it
 * goes to the back of the free queue when that reaches 0 (table order), and
 * its table entry becomes -1.  Logical positions do not move, so later
 * tokens keep their slots; decode reads -1 entries as empty blocks.  For a
 * window W, token = L + 1 - W (L tokens stored now) releases exactly what no
 * later decode can attend.  0 <= token <= length, else PKV_E_INVAL.
 * *n_released_out: table entries released by this call. */
pkv_status block_table_release_before(kv_pool* pool, int32_t seq, int32_t token,
                                      int32_t* n_released_out);

/* Copy a sequence's table (up to cap entries) and report its block count and
 * token length.  blocks_out may be NULL when cap == 0. */
pkv_status block_table_get(const kv_pool* pool, int32_t seq, int32_t* blocks_out,
                           int32_t cap, int32_t* n_blocks_out, int32_t* len_out);

/* Leading blocks shared by a batch: the largest k such that, for every
 * sequence in seqs, table entries 0 .. k-1 are the same physical blocks as
 * seqs[0]'s and all k blocks are full (k * block_size <= its length).  These
 * are the blocks forked sequences still hold in common (page "生成一个字…",
 * section "PagedAttention：…": a shared prefix is stored once, reference
 * counted).  n == 0 gives 0.  PKV_E_INVAL for an unknown id. */
pkv_status block_table_common_prefix(const kv_pool* pool, const int32_t* seqs, int32_t n,
                                     int32_t* blocks_out);

/* Dense export for the decode kernel: tables_out host int32 [n][max_blocks]
 * (row i = table of seqs[i], padded with -1), lens_out host int32 [n] (token
 * counts).  PKV_E_INVAL if a table has more than max_blocks entries. */
pkv_status block_table_export(const kv_pool* pool, const int32_t* seqs, int32_t n,
                              int32_t max_blocks, int32_t* tables_out, int32_t* lens_out);

/* ---- prefix cache (host only; page "第2章 KV Cache：模型内部的显存复用",
 *      chapter summary and section 2.4: a radix tree organises the prefixes
 *      of multi-turn conversations into a cache that later requests hit;
 *      page "生成一个字…", section "PagedAttention：…": shared blocks are
 *      stored once, reference counted) ----
 * A radix tree over token ids whose edges hold runs of whole blocks of one
 * pool.  Granularity is the block: only full blocks are cached or matched.
 * The cache holds one reference on each block it caches (so the blocks stay
 * allocated after the sequences that wrote them are freed) and never caches
 * the same tokens under the same prefix twice.  Every match or insert
 * touches the blocks on its path (one clock tick per call); eviction gives
 * back, one block at a time, the deepest block of the least recently touched
 * leaf whose block no sequence holds.  The pool must outlive the cache.  Not
 * thread-safe: calls on a pool and its cache are serialised by the caller. */
typedef struct kv_prefix_cache kv_prefix_cache;

pkv_status prefix_cache_create(kv_pool* pool, kv_prefix_cache** out);
/* Drops every reference the cache holds (in eviction order) and frees it. */
void prefix_cache_destroy(kv_prefix_cache* cache);
/* Longest cached prefix of tokens[0 .. n) in whole blocks.  Always creates a
 * new sequence (*seq_out) holding the matched blocks (one more reference
 * each, as a fork would) with length *matched_out = the matched tokens, a
 * multiple of block_size (0 on a miss).  The caller appends the rest of the
 * prompt to it.  PKV_E_INVAL for bad arguments; on failure nothing changes. */
pkv_status prefix_cache_match(kv_prefix_cache* cache, const int32_t* tokens, int32_t n,
                              int32_t* seq_out, int32_t* matched_out);
/* Caches the full blocks of seq that tokens[0 .. n) describe (the first
 * min(n, length) / block_size blocks, up to the first released entry).  Blocks
 * whose tokens are already cached under the same prefix are not added; the
 * rest get one reference from the cache.  tokens must be the tokens whose K/V
 * the sequence holds.  PKV_E_INVAL for an unknown id. */
pkv_status prefix_cache_insert(kv_prefix_cache* cache, int32_t seq, const int32_t* tokens, int32_t n);
/* Gives back up to n_blocks cached blocks that no sequence holds, least
 * recently used leaves first, deepest block first; *freed_out: how many went
 * back to the free queue (fewer when nothing else can be evicted). */
pkv_status prefix_cache_evict(kv_prefix_cache* cache, int32_t n_blocks, int32_t* freed_out);
/* Blocks the cache holds and tree nodes (edges). */
pkv_status prefix_cache_stats(const kv_prefix_cache* cache, int32_t* cached_blocks_out,
                              int32_t* nodes_out);

/* ---- device work ---- */

/* Whole-block copies for copy-on-write (page "生成一个字…", section
 * "PagedAttention：…"; page "AI 陪读顶会论文（三）", innovation 3): for each
 * pair, K and V of block dst in every layer become a byte copy of block src.
 * d_pairs: device array [n].  Pairs with an id outside [0, num_blocks) are
 * skipped; a dst must not also be a src in the same call. */
pkv_status kv_pool_copy_blocks(kv_pool* pool, const kv_block_copy* d_pairs, int32_t n,
                               pkv_stream stream);

/* Per-step metadata to the device (page "AI 陪读顶会论文（三）", section
 * "PagedAttention 的破局哲学": the kernel finds each sequence's blocks through
 * its block table, so the tables, lengths and new slots built on the host
 * must reach device memory before the step's kernels run).  Copies `bytes`
 * from h_src to d_dst in stream order, by a kernel on `stream` (no copy
 * engine, so no hand-off between hardware queues around the copy).
 * h_src: page-locked host memory (hipHostMalloc, or a torch tensor made with
 * pin_memory=True); [h_src, h_src + bytes) must lie inside one such
 * allocation.  d_dst: device memory, [d_dst, d_dst + bytes) inside one
 * allocation.  Both 8-byte aligned, bytes a multiple of 4, else PKV_E_INVAL.
 * The host must leave h_src unchanged until the copy has run (record an event
 * after this call and wait on it before rewriting the buffer). */
pkv_status kv_metadata_upload(void* d_dst, const void* h_src, size_t bytes, pkv_stream stream);

/* Write the new tokens' K and V into their slots of one layer (page
 * "AI 陪读顶会论文（三）", section "为什么自回归解码…必须使用 KV Cache").
 * d_k, d_v: device [n_tokens][num_kv_heads][head_dim] of src_dtype.
 * d_slots: device int64 [n_tokens] from block_table_append; a negative slot
 * or one >= num_blocks * block_size is skipped.
 * If src_dtype == the pool dtype the bits are copied.  For an FP8 pool,
 * src_dtype may be PKV_F32, PKV_F16 or PKV_BF16: each value x is widened to
 * fp32, multiplied in fp32 by inv_scale[layer][head][channel] and encoded to
 * E4M3 with round-to-nearest-even; magnitudes >= 448 and infinities saturate
 * to +-448, NaN becomes 0x7F.  Other combinations return PKV_E_DTYPE. */
pkv_status paged_kv_append(kv_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                           int32_t src_dtype, const int64_t* d_slots, int32_t n_tokens,
                           pkv_stream stream);

/* One decode step of a batch whose tables are resident on the device: row
 * i (0 <= i < n) gets one new token, the token of slots[i] (from
 * block_table_append_batch over the batch's sequences in row order).  Its K
 * and V are written as paged_kv_append writes them, and the same kernel
 * brings the row's metadata up to date: d_tables[i][d_lens[i] / block_size]
 * = slots[i] / block_size (a new block, or the block a copy-on-write made),
 * then d_lens[i] += 1 -- exactly the host block manager's table and length,
 * without exporting and uploading the whole tables each step (a4 done in
 * place; page "AI 陪读顶会论文（三）", section "PagedAttention 的破局哲学").
 * d_tables: device int32 [n][max_blocks], d_lens: device int32 [n], both
 * equal to the host state before the step (upload them once, e.g. with
 * block_table_export + kv_metadata_upload).  slots: int64 [n] in device
 * memory or in page-locked host memory (read directly by the kernel; keep it
 * unchanged until the step has run).  Copy-on-write pairs of the step must be
 * copied (kv_pool_copy_blocks) before.  A slot outside the pool, or a
 * position at or past max_blocks * block_size, leaves that row unchanged.
 * PKV_E_INVAL when a pointer does not lie in a suitable allocation. */
pkv_status paged_kv_append_step(kv_pool* pool, int32_t layer, const void* d_k, const void* d_v,
                                int32_t src_dtype, const int64_t* slots, int32_t n, int32_t* d_tables,
                                int32_t* d_lens, int32_t max_blocks, pkv_stream stream);

typedef struct {
  int32_t layer;
  int32_t batch;                /* B >= 0 */
  int32_t num_q_heads;          /* Hq, a multiple of num_kv_heads, Hq / Hkv <= 16 */
  int32_t max_blocks_per_seq;   /* row length of block_tables */
  int32_t sliding_window;       /* 0: off; W > 0: keys L-W .. L-1 only */
  int32_t num_splits;           /* <= 16384.  0: automatic; 1: single pass, one wavefront per
                                   (sequence, KV head), no workspace; n >= 2: the
                                   work units of all (KV head, sequence) pairs (a
                                   unit is max(block_size, 16 / 32 / 64) tokens for
                                   fp32 / fp16, bf16 / FP8 pools), laid end to end,
                                   are cut into n equal ranges, one per wavefront,
                                   and the pieces of a sequence split between ranges
                                   are combined by a log-sum-exp merge */
  const void* q;                /* device [B][Hq][head_dim], 16-byte aligned */
  int32_t q_dtype;              /* PKV_F32 for an fp32 pool, PKV_F16 for fp16,
                                   PKV_BF16 for bf16 and FP8 pools */
  int32_t* block_tables;        /* device int32 [B][max_blocks_per_seq]; written only by a
                                   fused append (below) */
  int32_t* context_lens;        /* device int32 [B]: tokens including the new one (with a
                                   fused append: the cached tokens before it; the call
                                   then adds one) */
  float scale;                  /* multiplies q.k; 1/sqrt(head_dim) by convention */
  void* out;                    /* device [B][Hq][head_dim], 16-byte aligned */
  int32_t out_dtype;            /* PKV_F32 (recommended), PKV_F16 or PKV_BF16 */
  void* workspace;              /* device, caller-owned, 256-byte aligned */
  size_t workspace_bytes;       /* >= paged_attention_workspace_size() */
  int32_t shared_prefix_blocks; /* 0: off.  k > 0: the first k table entries of
                                   every row are the same physical blocks as row
                                   0's (block_table_common_prefix gives the largest
                                   such k).  Those blocks are then read once for
                                   the whole batch by a prefix pass, which scores
                                   every query of a KV head against each of their
                                   K/V sub-tiles, and each sequence's own blocks
                                   from k on are read as usual; the two are joined
                                   by the log-sum-exp merge.  Same result as k = 0.
                                   Needs sliding_window == 0 (else
                                   PKV_E_UNSUPPORTED) and k <= max_blocks_per_seq;
                                   the workspace is then needed for every
                                   num_splits.  Page "生成一个字…", section
                                   "PagedAttention：…", and page "AI 陪读顶会论文（三）",
                                   innovation 3: a shared prefix is stored once;
                                   here it is also read once per call. */
  /* Fused append (optional; new_k == NULL: off).  The step's new token is
   * appended and attended in the same call (page "AI 陪读顶会论文（三）", section
   * "为什么自回归解码…必须使用 KV Cache": each step appends the new token's k, v
   * and its query attends every cached token, itself included).  Then
   * context_lens[b] = L counts the cached tokens before the new one, and the
   * call:
   *  - attends the L cached tokens and the new token (k, v from new_k, new_v,
   *    quantised like the pool for FP8; the window, if set, ends at the new
   *    token), combining the new token with the rest by the log-sum-exp merge;
   *  - writes the new token into the pool at new_slots[b] (as paged_kv_append
   *    does), block_tables[b][L / block_size] = new_slots[b] / block_size
   *    and context_lens[b] = L + 1, after every read of them.
   * new_slots[b] is the slot block_table_append gave (its copy-on-write
   * pairs copied first).  Every row's new token is attended.  A slot
   * outside the pool leaves the token unstored; such a slot, or
   * L / block_size not below max_blocks_per_seq, leaves the row's table
   * entry and length as they were.  The slots are read on the device while
   * the call runs.
   * Same result as paged_kv_append followed by paged_attention_decode.
   * The tables and lengths belong to the step, not to a layer: in a pool of
   * several layers, fuse the append into one call per step (the first
   * layer's), and let every later layer store its own token with
   * paged_kv_append and decode the L + 1 tokens. */
  const void* new_k;            /* device [B][Hkv][head_dim], 16-byte aligned */
  const void* new_v;            /* device [B][Hkv][head_dim], 16-byte aligned */
  int32_t new_dtype;            /* the pool's dtype, or f32 / f16 / bf16 into an FP8 pool */
  const int64_t* new_slots;     /* device or page-locked host [B] */
} paged_decode_args;

/* Workspace paged_attention_decode needs for these arguments (0 for a single
 * pass).  For num_splits == 0 this queries the current device.
 * The workspace holds the partial results of sequences whose blocks are
 * split over several wavefronts; it needs no initialisation.  One workspace
 * serves one call at a time: calls that may overlap (other streams)
 * need their own. */
pkv_status paged_attention_workspace_size(const kv_pool* pool, const paged_decode_args* args,
                                          size_t* bytes_out);

/* Decode attention over the paged cache (page "AI 陪读顶会论文（三）", section
 * "为什么自回归解码…必须使用 KV Cache", the attention equation; GQA from page
 * "生成一个字…", section "显存账本"):
 *   for every sequence b and query head h, with G = Hq / Hkv, KV head
 *   g = h / G, L = context_lens[b] and lo = max(0, L - W) if a window W is
 *   set (else 0):
 *     out[b][h] = sum_{j=lo}^{L-1} softmax_j(scale * q[b][h] . k_j) v_j
 *   where token j of sequence b is read from physical block
 *   block_tables[b][j / block_size] at offset j % block_size.
 * FP8 pools are dequantised as code value * per-channel scale.  L = 0 (or an
 * empty window) gives zeros.  Table entries outside [0, num_blocks) are read
 * as empty blocks (their tokens are skipped) and L is clamped to
 * max_blocks_per_seq * block_size, so no access leaves the buffers. */
pkv_status paged_attention_decode(const kv_pool* pool, const paged_decode_args* args,
                                  pkv_stream stream);

/* Size of the library's static decode workspace (64 MiB): device memory that
 * every GPU the library runs on holds from the first use of the library's
 * kernels until the process ends. */
#define PKV_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

/* paged_attention_decode without a caller-owned workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same operation and result as
 * paged_attention_decode; the split-K partials and merge records live in a
 * static device array of PKV_STATIC_WORKSPACE_BYTES per GPU.  This call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine);
 * on its first use on a device it looks up that device's array address.
 *  - args->workspace must be NULL and args->workspace_bytes 0 (else
 *    PKV_E_INVAL).
 *  - PKV_E_UNSUPPORTED, before any launch, when the call needs more than
 *    PKV_STATIC_WORKSPACE_BYTES of workspace (paged_attention_workspace_size
 *    gives the need; e.g. num_splits far above the automatic 4 per CU with a
 *    large query group): use paged_attention_decode then.
 *  - Every call on one GPU shares that GPU's array, which keeps the last
 *    call's contents (the decode rewrites what it reads, so nothing needs
 *    clearing).  Calls that may overlap on one GPU (different streams, or
 *    host threads racing on one stream) race on the array: order them. */
pkv_status paged_attention_decode_static(const kv_pool* pool, const paged_decode_args* args,
                                         pkv_stream stream);

/* paged_attention_decode, timed by its own kernels (same operation, same
 * pages).  kernel_events: host array of four hipEvent_t created with timing
 * enabled (caller-owned): [0] and [1] are recorded when the attention kernel
 * starts and ends (with a shared prefix, [0] when the prefix pass before it
 * starts), [2] and [3] when the log-sum-exp merge kernel starts and ends
 * (hipExtLaunchKernelGGL), so each elapsed time is the device duration of
 * those kernels.  *n_kernels_out (may be NULL): 1 when the call ran
 * no merge kernel (then [2] and [3] are left as they were), else 2.
 * PKV_E_INVAL if kernel_events or one of its entries is NULL.  Recording an
 * event makes the runtime finish the kernel with a system-scope release, which
 * adds a few microseconds of idle time after it: time a sample of calls. */
pkv_status paged_attention_decode_timed(const kv_pool* pool, const paged_decode_args* args,
                                        pkv_stream stream, void* const* kernel_events,
                                        int32_t* n_kernels_out);

/* Measurement helper, not part of the method: reads [d_buf, d_buf + bytes)
 * of device memory once, with the 16-byte streaming loads the decode uses for
 * K and V, so that the time of this call is the achievable HBM read rate that
 * the decode's own rate can be compared with (the decode is bound by HBM
 * bandwidth: page "生成一个字…", section "显存账本", every generated token
 * reads the whole KV cache).  d_buf: device, 16-byte aligned, bytes a
 * multiple of 16, inside one allocation; d_sink: device, 4 bytes, written
 * only when the XOR of what one thread read equals tag.  Asynchronous on
 * stream.  PKV_E_INVAL on a bad pointer or size. */
pkv_status pkv_hbm_read_probe(const void* d_buf, size_t bytes, uint32_t* d_sink, uint32_t tag,
                              pkv_stream stream);

/* Message describing the last failure on the calling thread ("" if none). */
const char* pkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
