// Block tables of a paged KV pool: free-block queue, per-sequence tables,
// reference counts, on-demand append with copy-on-write, fork and free.
//
// Page "生成一个字，为什么要背一整本账", section
// "PagedAttention：把操作系统的老智慧搬进推理引擎": blocks of a fixed number of
// tokens, mapped through a per-sequence table, taken on demand, shared
// prefixes stored once with reference counts and copied on write where
// sequences diverge.  Page "AI 陪读顶会论文（三）", section
// "PagedAttention 的破局哲学": tokens 1-16 in logical block 0, 17-32 in
// block 1, ...; the second block is taken when the 17th token arrives.
//
// Policy where the pages are silent: tokens counted from 0; FIFO free queue
// seeded from free_order; blocks released in table order; lazy copy-on-write
// of a shared, partly filled last block at the first append into it; every
// mutating call either fully succeeds or changes nothing.
#include <algorithm>
#include <cstring>
#include <new>
#include <unordered_map>

#include "pool_internal.h"

namespace pkv {

static thread_local std::string g_last_error;

void set_error(const std::string& msg) { g_last_error = msg; }

pkv_status fail(pkv_status code, const std::string& msg) {
  g_last_error = msg;
  return code;
}

int elem_bytes(int32_t dtype) {
  switch (dtype) {
    case PKV_F32: return 4;
    case PKV_F16: return 2;
    case PKV_BF16: return 2;
    case PKV_FP8_E4M3: return 1;
    default: return 0;
  }
}

static inline int32_t pop_free(kv_pool* p) {
  int32_t b = p->ring[p->head];
  p->head = (p->head + 1) % (int64_t)p->ring.size();
  p->count--;
  return b;
}

static inline void push_free(kv_pool* p, int32_t b) {
  p->ring[(p->head + p->count) % (int64_t)p->ring.size()] = b;
  p->count++;
}

// Blocks one append of n tokens to s needs, given an effective reference
// count of its last block.
static inline int64_t blocks_needed(const Sequence& s, int64_t n, int32_t bs,
                                    int32_t last_ref, bool* cow) {
  const int64_t before = (s.len + bs - 1) / bs;
  const int64_t after = (s.len + n + bs - 1) / bs;
  *cow = n > 0 && (s.len % bs) != 0 && last_ref > 1;
  return (after - before) + (*cow ? 1 : 0);
}

// Room for `more` table entries, growing geometrically so that a sequence
// that gains one block at a time reallocates O(log n) times.
static inline void reserve_more(std::vector<int32_t>& t, int64_t more) {
  const size_t want = t.size() + (size_t)more;
  if (t.capacity() < want) t.reserve(std::max<size_t>({want, 2 * t.capacity(), 16}));
}

// Freed sequences whose map nodes are kept for reuse by forks, and the
// largest table (entries) a kept node may hold on to: at most 4 MiB of host
// memory stays with the pool this way.
static constexpr size_t kSpareNodes = 1024;
static constexpr size_t kSpareTableCap = 1024;

// Resolves a batch of sequence ids into p->batch, rejecting unknown and
// repeated ids.
static pkv_status resolve_batch(kv_pool* p, const int32_t* seqs, int32_t n) {
  const uint64_t stamp = ++p->stamp;
  p->batch.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id in batch");
    if (it->second.mark == stamp) return fail(PKV_E_INVAL, "duplicate sequence in batch");
    it->second.mark = stamp;
    p->batch[i] = &it->second;
  }
  return PKV_OK;
}

// Freed sequence: its node goes to the spare list while there is room
// (reserved, so this never allocates), else it is released.
static void retire_sequence(kv_pool* p, int32_t id) {
  auto nh = p->seqs.extract(id);
  if (nh.empty() || p->spare.size() >= p->spare.capacity()) return;
  Sequence& s = nh.mapped();
  if (s.table.capacity() > kSpareTableCap) std::vector<int32_t>().swap(s.table);
  s.table.clear();
  s.len = 0;
  s.mark = 0;
  p->spare.push_back(std::move(nh));
}

// Performs an append whose block needs were checked; cannot fail.
static void do_append(kv_pool* p, Sequence& s, int64_t n, int64_t* slots,
                      kv_block_copy* cow, int32_t* n_cow) {
  const int32_t bs = p->desc.block_size;
  const int64_t start = s.len;
  for (int64_t pos = start; pos < start + n; ++pos) {
    if (pos % bs == 0) {
      int32_t b = pop_free(p);
      p->refcount[b] = 1;
      s.table.push_back(b);
    } else if (pos == start && p->refcount[s.table[pos / bs]] > 1) {
      int32_t old = s.table[pos / bs];
      int32_t nw = pop_free(p);
      p->refcount[old] -= 1;
      p->refcount[nw] = 1;
      s.table[pos / bs] = nw;
      cow[*n_cow].src = old;
      cow[*n_cow].dst = nw;
      (*n_cow)++;
    }
    slots[pos - start] = (int64_t)s.table[pos / bs] * bs + pos % bs;
  }
  s.len = start + n;
}

void block_ref(kv_pool* p, int32_t b) { p->refcount[b] += 1; }

void block_unref(kv_pool* p, int32_t b) {
  p->refcount[b] -= 1;
  if (p->refcount[b] == 0) push_free(p, b);
}

int32_t adopt_sequence(kv_pool* p, const std::vector<int32_t>& blocks, int64_t len) {
  Sequence s;
  s.table = blocks;     // may throw: nothing changed yet
  s.len = len;
  const int32_t id = p->next_id;
  p->seqs.emplace(id, std::move(s));
  for (int32_t b : blocks) p->refcount[b] += 1;
  p->next_id++;
  return id;
}

}  // namespace pkv

using namespace pkv;

#define PKV_GUARD_BEGIN try {
#define PKV_GUARD_END                                                   \
  }                                                                     \
  catch (const std::bad_alloc&) {                                       \
    return fail(PKV_E_INTERNAL, "host allocation failed");              \
  }                                                                     \
  catch (...) {                                                         \
    return fail(PKV_E_INTERNAL, "unexpected internal error");           \
  }

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

pkv_status kv_pool_cache_bytes(const kv_pool_desc* d, size_t* bytes_out) {
  if (!d || !bytes_out) return fail(PKV_E_INVAL, "null argument");
  const int eb = elem_bytes(d->kv_dtype);
  if (!eb) return fail(PKV_E_DTYPE, "unknown kv_dtype");
  if (d->num_layers <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 ||
      d->block_size <= 0 || d->num_blocks <= 0)
    return fail(PKV_E_INVAL, "sizes must be positive");
  *bytes_out = (size_t)d->num_layers * (size_t)d->num_blocks * (size_t)d->num_kv_heads *
               (size_t)d->block_size * (size_t)d->head_dim * (size_t)eb;
  return PKV_OK;
}

pkv_status kv_pool_create(const kv_pool_desc* d, kv_pool** out) {
  PKV_GUARD_BEGIN
  if (!d || !out) return fail(PKV_E_INVAL, "null argument");
  *out = nullptr;
  size_t bytes = 0;
  pkv_status st = kv_pool_cache_bytes(d, &bytes);
  if (st != PKV_OK) return st;
  const bool fp8 = d->kv_dtype == PKV_FP8_E4M3;
  const bool any_scale = d->k_scale || d->v_scale || d->k_inv_scale || d->v_inv_scale;
  const bool all_scale = d->k_scale && d->v_scale && d->k_inv_scale && d->v_inv_scale;
  if (fp8 && !all_scale) return fail(PKV_E_INVAL, "FP8 pool needs k/v scale and inv_scale");
  if (!fp8 && any_scale) return fail(PKV_E_INVAL, "scales are only for FP8 pools");
  if ((d->k_cache == nullptr) != (d->v_cache == nullptr))
    return fail(PKV_E_INVAL, "k_cache and v_cache must both be set or both be NULL");
  kv_pool* p = new kv_pool();
  p->desc = *d;
  p->desc.free_order = nullptr;
  const int32_t nb = d->num_blocks;
  p->ring.resize(nb);
  p->refcount.assign(nb, 0);
  p->spare.reserve(kSpareNodes);
  if (d->free_order) {
    std::vector<char> seen(nb, 0);
    for (int32_t i = 0; i < nb; ++i) {
      int32_t b = d->free_order[i];
      if (b < 0 || b >= nb || seen[b]) {
        delete p;
        return fail(PKV_E_INVAL, "free_order is not a permutation of 0..num_blocks-1");
      }
      seen[b] = 1;
      p->ring[i] = b;
    }
  } else {
    for (int32_t i = 0; i < nb; ++i) p->ring[i] = i;
  }
  p->head = 0;
  p->count = nb;
  *out = p;
  return PKV_OK;
  PKV_GUARD_END
}

void kv_pool_destroy(kv_pool* p) { delete p; }

pkv_status kv_pool_num_free(const kv_pool* p, int32_t* out) {
  if (!p || !out) return fail(PKV_E_INVAL, "null argument");
  *out = (int32_t)p->count;
  return PKV_OK;
}

pkv_status kv_pool_refcount(const kv_pool* p, int32_t block, int32_t* out) {
  if (!p || !out) return fail(PKV_E_INVAL, "null argument");
  if (block < 0 || block >= p->desc.num_blocks) return fail(PKV_E_INVAL, "block id out of range");
  *out = p->refcount[block];
  return PKV_OK;
}

pkv_status kv_pool_free_list(const kv_pool* p, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!p || !n_out || (cap > 0 && !out) || cap < 0) return fail(PKV_E_INVAL, "bad argument");
  const int64_t n = std::min<int64_t>(cap, p->count);
  for (int64_t i = 0; i < n; ++i) out[i] = p->ring[(p->head + i) % (int64_t)p->ring.size()];
  *n_out = (int32_t)p->count;
  return PKV_OK;
}

pkv_status block_table_alloc(kv_pool* p, int32_t* seq_out) {
  PKV_GUARD_BEGIN
  if (!p || !seq_out) return fail(PKV_E_INVAL, "null argument");
  if (p->next_id == INT32_MAX) return fail(PKV_E_INVAL, "sequence ids exhausted");
  const int32_t id = p->next_id;
  p->seqs.emplace(id, Sequence());
  p->next_id++;
  *seq_out = id;
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status block_table_append(kv_pool* p, int32_t seq, int32_t n_tokens, int64_t* slots_out,
                              kv_block_copy* cow_out, int32_t* n_cow_out) {
  PKV_GUARD_BEGIN
  if (!p || !n_cow_out || !cow_out || (n_tokens > 0 && !slots_out))
    return fail(PKV_E_INVAL, "null argument");
  if (n_tokens < 0) return fail(PKV_E_INVAL, "n_tokens must be >= 0");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id");
  Sequence& s = it->second;
  if (s.len + n_tokens > (int64_t)INT32_MAX) return fail(PKV_E_INVAL, "sequence too long");
  const int32_t bs = p->desc.block_size;
  const int32_t last_ref = (s.len % bs) ? p->refcount[s.table.back()] : 0;
  bool cow = false;
  const int64_t need = blocks_needed(s, n_tokens, bs, last_ref, &cow);
  // the table grows by at most `need` entries: reserve first so that the
  // mutation below cannot throw
  reserve_more(s.table, need);
  if (need > p->count) return fail(PKV_E_OOM, "not enough free blocks");
  *n_cow_out = 0;
  do_append(p, s, n_tokens, slots_out, cow_out, n_cow_out);
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status block_table_append_batch(kv_pool* p, const int32_t* seqs, int32_t n,
                                    int64_t* slots_out, kv_block_copy* cow_out,
                                    int32_t* n_cow_out) {
  PKV_GUARD_BEGIN
  if (!p || !n_cow_out || n < 0 || (n > 0 && (!seqs || !slots_out || !cow_out)))
    return fail(PKV_E_INVAL, "bad argument");
  const int32_t bs = p->desc.block_size;
  pkv_status st = resolve_batch(p, seqs, n);
  if (st != PKV_OK) return st;
  if (p->ref_delta.size() != (size_t)p->desc.num_blocks) p->ref_delta.assign(p->desc.num_blocks, 0);
  // dry run: count blocks with the reference counts the earlier sequences of
  // the batch leave behind (a shared last block copied by one of them has one
  // holder fewer for the next)
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    Sequence& s = *p->batch[i];
    if (s.len + 1 > (int64_t)INT32_MAX) {
      need = -1;
      break;
    }
    int32_t last_ref = 0;
    if (s.len % bs) {
      const int32_t last = s.table.back();
      last_ref = p->refcount[last] + p->ref_delta[last];
    }
    bool cow = false;
    need += blocks_needed(s, 1, bs, last_ref, &cow);
    if (cow) {
      if (p->ref_delta[s.table.back()] == 0) p->touched.push_back(s.table.back());
      p->ref_delta[s.table.back()] -= 1;
    }
  }
  for (int32_t b : p->touched) p->ref_delta[b] = 0;
  p->touched.clear();
  if (need < 0) return fail(PKV_E_INVAL, "sequence too long");
  if (need > p->count) return fail(PKV_E_OOM, "not enough free blocks");
  // only a sequence at a block boundary pushes a table entry (a copy-on-write
  // replaces the last one): reserve for those, so that a fresh fork (table
  // capacity == size) is not reallocated for nothing
  for (int32_t i = 0; i < n; ++i)
    if (p->batch[i]->len % bs == 0) reserve_more(p->batch[i]->table, 1);
  *n_cow_out = 0;
  for (int32_t i = 0; i < n; ++i) do_append(p, *p->batch[i], 1, slots_out + i, cow_out, n_cow_out);
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status block_table_fork(kv_pool* p, int32_t parent, int32_t* child_out) {
  PKV_GUARD_BEGIN
  if (!p || !child_out) return fail(PKV_E_INVAL, "null argument");
  auto it = p->seqs.find(parent);
  if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id");
  if (p->next_id == INT32_MAX) return fail(PKV_E_INVAL, "sequence ids exhausted");
  Sequence child = it->second;  // copy first: may throw, state untouched
  const int32_t id = p->next_id;
  auto res = p->seqs.emplace(id, std::move(child));
  for (int32_t b : res.first->second.table)
    if (b >= 0) p->refcount[b] += 1;
  p->next_id++;
  *child_out = id;
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status block_table_free(kv_pool* p, int32_t seq) {
  PKV_GUARD_BEGIN
  if (!p) return fail(PKV_E_INVAL, "null argument");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id");
  for (int32_t b : it->second.table) {
    if (b < 0) continue;
    p->refcount[b] -= 1;
    if (p->refcount[b] == 0) push_free(p, b);
  }
  retire_sequence(p, seq);
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status block_table_release_before(kv_pool* p, int32_t seq, int32_t token, int32_t* n_released_out) {
  if (!p || !n_released_out) return fail(PKV_E_INVAL, "null argument");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id");
  Sequence& s = it->second;
  if (token < 0 || token > s.len) return fail(PKV_E_INVAL, "token must lie in [0, length]");
  int32_t n = 0;
  const int64_t nblk = token / p->desc.block_size;
  for (int64_t i = 0; i < nblk; ++i) {
    const int32_t b = s.table[i];
    if (b < 0) continue;
    p->refcount[b] -= 1;
    if (p->refcount[b] == 0) push_free(p, b);
    s.table[i] = -1;
    ++n;
  }
  *n_released_out = n;
  return PKV_OK;
}

pkv_status block_table_fork_batch(kv_pool* p, const int32_t* parents, int32_t n, int32_t* children_out) {
  PKV_GUARD_BEGIN
  if (!p || n < 0 || (n > 0 && (!parents || !children_out))) return fail(PKV_E_INVAL, "bad argument");
  if ((int64_t)p->next_id + n > (int64_t)INT32_MAX) return fail(PKV_E_INVAL, "sequence ids exhausted");
  std::vector<const Sequence*> par(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = p->seqs.find(parents[i]);
    if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id in batch");
    par[i] = &it->second;
  }
  // every child's node and table first, from the spare nodes where there are
  // any (a failure here leaves the pool as it was: nodes not inserted are
  // released, or go back to the spare list)
  const int32_t id0 = p->next_id;
  std::vector<decltype(p->spare)::value_type> nodes;
  nodes.reserve(n);
  try {
    for (int32_t i = 0; i < n; ++i) {
      decltype(p->spare)::value_type nh;
      if (!p->spare.empty()) {
        nh = std::move(p->spare.back());
        p->spare.pop_back();
      } else {
        decltype(p->seqs) one;
        one.emplace(0, Sequence());
        nh = one.extract(one.begin());
      }
      nodes.push_back(std::move(nh));   // within the reserved room
      Sequence& c = nodes.back().mapped();
      nodes.back().key() = id0 + i;
      c.table.assign(par[i]->table.begin(), par[i]->table.end());
      c.len = par[i]->len;
      c.mark = 0;
    }
    p->seqs.reserve(p->seqs.size() + n);
  } catch (...) {
    while (!nodes.empty() && p->spare.size() < p->spare.capacity()) {
      p->spare.push_back(std::move(nodes.back()));
      nodes.pop_back();
    }
    throw;
  }
  // no allocation from here: the nodes exist and the buckets are reserved
  for (int32_t i = 0; i < n; ++i) {
    auto res = p->seqs.insert(std::move(nodes[i]));
    for (int32_t b : res.position->second.table)
      if (b >= 0) p->refcount[b] += 1;
    children_out[i] = id0 + i;
  }
  p->next_id += n;
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status block_table_free_batch(kv_pool* p, const int32_t* seqs, int32_t n) {
  PKV_GUARD_BEGIN
  if (!p || n < 0 || (n > 0 && !seqs)) return fail(PKV_E_INVAL, "bad argument");
  pkv_status st = resolve_batch(p, seqs, n);
  if (st != PKV_OK) return st;
  for (int32_t i = 0; i < n; ++i) {
    for (int32_t b : p->batch[i]->table) {
      if (b < 0) continue;
      p->refcount[b] -= 1;
      if (p->refcount[b] == 0) push_free(p, b);
    }
  }
  for (int32_t i = 0; i < n; ++i) retire_sequence(p, seqs[i]);
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status block_table_get(const kv_pool* p, int32_t seq, int32_t* blocks_out, int32_t cap,
                           int32_t* n_blocks_out, int32_t* len_out) {
  if (!p || !n_blocks_out || !len_out || cap < 0 || (cap > 0 && !blocks_out))
    return fail(PKV_E_INVAL, "bad argument");
  auto it = p->seqs.find(seq);
  if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id");
  const auto& t = it->second.table;
  const size_t n = std::min<size_t>(cap, t.size());
  if (n) std::memcpy(blocks_out, t.data(), n * sizeof(int32_t));
  *n_blocks_out = (int32_t)t.size();
  *len_out = (int32_t)it->second.len;
  return PKV_OK;
}

pkv_status block_table_common_prefix(const kv_pool* p, const int32_t* seqs, int32_t n, int32_t* blocks_out) {
  if (!p || !blocks_out || n < 0 || (n > 0 && !seqs)) return fail(PKV_E_INVAL, "bad argument");
  PKV_GUARD_BEGIN
  p->batch.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = const_cast<kv_pool*>(p)->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id");
    p->batch[i] = &it->second;
  }
  int64_t k = 0;
  if (n > 0) {
    const Sequence& s0 = *p->batch[0];
    // row 0's leading valid entries
    k = 0;
    while (k < (int64_t)s0.table.size() && s0.table[k] >= 0) ++k;
    for (int32_t i = 0; i < n && k > 0; ++i) {
      const Sequence& s = *p->batch[i];
      k = std::min<int64_t>(k, s.len / p->desc.block_size);   // full blocks only
      k = std::min<int64_t>(k, (int64_t)s.table.size());
      // whole common run equal (the usual case for forks): one memcmp
      if (k > 0 && std::memcmp(s.table.data(), s0.table.data(), (size_t)k * sizeof(int32_t)) == 0) continue;
      int64_t j = 0;
      while (j < k && s.table[j] == s0.table[j]) ++j;
      k = j;
    }
  }
  *blocks_out = (int32_t)k;
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status block_table_export(const kv_pool* p, const int32_t* seqs, int32_t n,
                              int32_t max_blocks, int32_t* tables_out, int32_t* lens_out) {
  if (!p || n < 0 || max_blocks < 0 ||
      (n > 0 && (!seqs || !lens_out || (max_blocks > 0 && !tables_out))))
    return fail(PKV_E_INVAL, "bad argument");
  PKV_GUARD_BEGIN
  p->batch.resize(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = const_cast<kv_pool*>(p)->seqs.find(seqs[i]);
    if (it == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id");
    if ((int64_t)it->second.table.size() > max_blocks)
      return fail(PKV_E_INVAL, "table longer than max_blocks");
    p->batch[i] = &it->second;
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& t = p->batch[i]->table;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    std::copy(t.begin(), t.end(), row);
    std::fill(row + t.size(), row + max_blocks, -1);
    lens_out[i] = (int32_t)p->batch[i]->len;
  }
  return PKV_OK;
  PKV_GUARD_END
}

}  // extern "C"
