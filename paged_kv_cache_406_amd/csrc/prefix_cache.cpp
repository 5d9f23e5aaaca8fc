// Prefix cache: a radix tree over token ids whose edges hold runs of whole
// KV blocks of a pool, so that a new request whose prompt starts like an
// earlier one (the next turn of a conversation, a shared system prompt)
// takes those blocks instead of computing and storing them again.
//
// Page "第2章 KV Cache：模型内部的显存复用" (chapter summary and section 2.4):
// a radix tree organises the prefixes of multi-turn conversations into a
// cache that later requests hit.  Page "生成一个字，为什么要背一整本账",
// section "PagedAttention：把操作系统的老智慧搬进推理引擎": shared prefix
// blocks are stored once and reference counted.  The pages give no more than
// that; the rules below are the plainest ones that fit paged blocks:
//
//  * Granularity is the block: an edge label is a multiple of block_size
//    tokens, and only full blocks are cached or matched (a partly filled
//    block would be written again).
//  * The tree holds one reference on every block it caches; a matched
//    request gets a new sequence holding the matched blocks (one more
//    reference each), exactly like a fork.
//  * A block whose tokens are already cached under the same prefix is not
//    cached twice: the tree keeps the block it has.
//  * Every match or insert touches the blocks on its path (one clock tick per
//    call).  A match that ends inside an edge splits it there, so exactly the
//    matched blocks are touched.
//  * Eviction takes, one block at a time, the deepest block of the least
//    recently touched leaf whose block only the tree still holds, and gives
//    it back to the pool.  (Leaves touched by the same call lie on one path,
//    so the least recently touched leaf is unique.)  Destroying the cache
//    drops its references in the same order, whoever else holds the blocks.
#include <algorithm>
#include <map>
#include <memory>
#include <new>
#include <vector>

#include "pool_internal.h"

using pkv::fail;

namespace {

struct Node {
  std::vector<int32_t> tokens;   // edge label, a multiple of block_size tokens
  std::vector<int32_t> blocks;   // one physical block per block_size tokens
  std::map<std::vector<int32_t>, std::unique_ptr<Node>> kids;  // keyed by the first block's tokens
  Node* parent = nullptr;
  uint64_t last_use = 0;         // clock of the last call that touched it
};

}  // namespace

struct kv_prefix_cache {
  kv_pool* pool = nullptr;
  Node root;
  uint64_t clock = 0;
  int64_t cached_blocks = 0;
};

namespace {

std::vector<int32_t> key_of(const int32_t* t, int32_t bs) { return std::vector<int32_t>(t, t + bs); }

// Splits `n` after its first k blocks (0 < k < blocks): the upper part keeps
// the key in the parent and the first k blocks; the rest becomes its only
// child.  Returns the upper part.
Node* split(Node* n, size_t k, int32_t bs) {
  Node* parent = n->parent;
  auto it = parent->kids.find(key_of(n->tokens.data(), bs));
  std::unique_ptr<Node> low = std::move(it->second);
  auto up = std::make_unique<Node>();
  up->tokens.assign(low->tokens.begin(), low->tokens.begin() + k * bs);
  up->blocks.assign(low->blocks.begin(), low->blocks.begin() + k);
  up->last_use = low->last_use;
  up->parent = parent;
  low->tokens.erase(low->tokens.begin(), low->tokens.begin() + k * bs);
  low->blocks.erase(low->blocks.begin(), low->blocks.begin() + k);
  low->parent = up.get();
  std::vector<int32_t> low_key = key_of(low->tokens.data(), bs);
  up->kids.emplace(std::move(low_key), std::move(low));
  Node* res = up.get();
  it->second = std::move(up);
  return res;
}

// Leaf with the smallest last_use (optionally only those whose deepest
// block has no holder but the tree); nullptr if none.
Node* oldest_leaf(Node* n, const kv_pool* p, bool only_unheld) {
  Node* best = nullptr;
  std::vector<Node*> stack{n};
  while (!stack.empty()) {
    Node* x = stack.back();
    stack.pop_back();
    if (x->kids.empty()) {
      if (x->parent && !x->blocks.empty() && (!only_unheld || p->refcount[x->blocks.back()] == 1) &&
          (!best || x->last_use < best->last_use))
        best = x;
      continue;
    }
    for (auto& kv : x->kids) stack.push_back(kv.second.get());
  }
  return best;
}

// Drops the tree's reference on the deepest block of leaf x; removes x when
// it has no block left.
void drop_last(kv_prefix_cache* c, Node* x) {
  const int32_t bs = c->pool->desc.block_size;
  const int32_t b = x->blocks.back();
  x->blocks.pop_back();
  x->tokens.resize(x->tokens.size() - bs);
  c->cached_blocks--;
  pkv::block_unref(c->pool, b);
  if (x->blocks.empty()) {
    Node* parent = x->parent;
    for (auto it = parent->kids.begin(); it != parent->kids.end(); ++it)
      if (it->second.get() == x) {
        parent->kids.erase(it);
        break;
      }
  }
}

int64_t count_nodes(const Node& n) {
  int64_t k = 0;
  for (const auto& kv : n.kids) k += 1 + count_nodes(*kv.second);
  return k;
}

}  // namespace

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

pkv_status prefix_cache_create(kv_pool* pool, kv_prefix_cache** out) {
  PKV_GUARD_BEGIN
  if (!pool || !out) return fail(PKV_E_INVAL, "null argument");
  auto* c = new kv_prefix_cache();
  c->pool = pool;
  *out = c;
  return PKV_OK;
  PKV_GUARD_END
}

void prefix_cache_destroy(kv_prefix_cache* c) {
  if (!c) return;
  while (Node* x = oldest_leaf(&c->root, c->pool, false)) drop_last(c, x);
  delete c;
}

pkv_status prefix_cache_match(kv_prefix_cache* c, const int32_t* tokens, int32_t n, int32_t* seq_out,
                              int32_t* matched_out) {
  PKV_GUARD_BEGIN
  if (!c || !seq_out || !matched_out || n < 0 || (n > 0 && !tokens)) return fail(PKV_E_INVAL, "bad argument");
  kv_pool* p = c->pool;
  if (p->next_id == INT32_MAX) return fail(PKV_E_INVAL, "sequence ids exhausted");
  const int32_t bs = p->desc.block_size;
  std::vector<int32_t> blocks;
  std::vector<Node*> path;
  Node* node = &c->root;
  int64_t pos = 0;
  while (pos + bs <= n) {
    auto it = node->kids.find(key_of(tokens + pos, bs));
    if (it == node->kids.end()) break;
    Node* child = it->second.get();
    size_t k = 0;
    while (k < child->blocks.size() && pos + bs <= n &&
           std::equal(tokens + pos, tokens + pos + bs, child->tokens.begin() + k * bs)) {
      blocks.push_back(child->blocks[k]);
      pos += bs;
      ++k;
    }
    // a match that ends inside an edge splits it there (the cached content
    // does not change), so that only the matched blocks are touched
    const bool partial = k < child->blocks.size();
    if (partial) child = split(child, k, bs);
    path.push_back(child);
    if (partial) break;
    node = child;
  }
  const int32_t seq = pkv::adopt_sequence(p, blocks, pos);   // may throw: nothing touched yet
  c->clock++;
  for (Node* x : path) x->last_use = c->clock;
  *seq_out = seq;
  *matched_out = (int32_t)pos;
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status prefix_cache_insert(kv_prefix_cache* c, int32_t seq, const int32_t* tokens, int32_t n) {
  PKV_GUARD_BEGIN
  if (!c || n < 0 || (n > 0 && !tokens)) return fail(PKV_E_INVAL, "bad argument");
  kv_pool* p = c->pool;
  auto sit = p->seqs.find(seq);
  if (sit == p->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence id");
  const pkv::Sequence& s = sit->second;
  const int32_t bs = p->desc.block_size;
  // full blocks of the sequence that the given tokens describe, up to the
  // first released (-1) entry
  int64_t nfull = std::min<int64_t>(n, s.len) / bs;
  nfull = std::min<int64_t>(nfull, (int64_t)s.table.size());
  for (int64_t b = 0; b < nfull; ++b)
    if (s.table[b] < 0) {
      nfull = b;
      break;
    }
  c->clock++;
  Node* node = &c->root;
  int64_t b = 0;
  while (b < nfull) {
    auto it = node->kids.find(key_of(tokens + b * bs, bs));
    if (it == node->kids.end()) {
      auto leaf = std::make_unique<Node>();
      leaf->tokens.assign(tokens + b * bs, tokens + nfull * bs);
      leaf->blocks.assign(s.table.begin() + b, s.table.begin() + nfull);
      leaf->last_use = c->clock;
      leaf->parent = node;
      std::vector<int32_t> key = key_of(tokens + b * bs, bs);
      node->kids.emplace(std::move(key), std::move(leaf));
      for (int64_t k = b; k < nfull; ++k) pkv::block_ref(p, s.table[k]);
      c->cached_blocks += nfull - b;
      break;
    }
    Node* child = it->second.get();
    size_t k = 0;
    while (k < child->blocks.size() && b < nfull &&
           std::equal(tokens + b * bs, tokens + (b + 1) * bs, child->tokens.begin() + k * bs)) {
      ++k;
      ++b;
    }
    if (k < child->blocks.size()) child = split(child, k, bs);
    child->last_use = c->clock;
    node = child;
  }
  return PKV_OK;
  PKV_GUARD_END
}

pkv_status prefix_cache_evict(kv_prefix_cache* c, int32_t n_blocks, int32_t* freed_out) {
  if (!c || !freed_out || n_blocks < 0) return fail(PKV_E_INVAL, "bad argument");
  int32_t freed = 0;
  while (freed < n_blocks) {
    Node* x = oldest_leaf(&c->root, c->pool, true);
    if (!x) break;
    drop_last(c, x);
    ++freed;
  }
  *freed_out = freed;
  return PKV_OK;
}

pkv_status prefix_cache_stats(const kv_prefix_cache* c, int32_t* cached_blocks_out, int32_t* nodes_out) {
  if (!c || !cached_blocks_out || !nodes_out) return fail(PKV_E_INVAL, "null argument");
  *cached_blocks_out = (int32_t)c->cached_blocks;
  *nodes_out = (int32_t)count_nodes(c->root);
  return PKV_OK;
}

}  // extern "C"
