// Host-side state of a paged KV pool, shared by the block-table code
// (pool.cpp) and the device launch code (kernels.hip).
#pragma once

#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace pkv {

struct Sequence {
  std::vector<int32_t> table;  // logical block i -> physical block id
  int64_t len = 0;             // tokens stored
  uint64_t mark = 0;           // batch calls: set to the call's stamp when seen
};

}  // namespace pkv

struct kv_pool {
  kv_pool_desc desc;                 // copy; free_order cleared after use
  // free-block FIFO as a ring buffer over num_blocks entries
  std::vector<int32_t> ring;
  int64_t head = 0;
  int64_t count = 0;
  std::vector<int32_t> refcount;
  std::unordered_map<int32_t, pkv::Sequence> seqs;
  // map nodes of freed sequences, tables cleared but still allocated, reused
  // by forks: a steady fork/free loop allocates nothing (capacity fixed at
  // creation, so keeping a node never allocates)
  std::vector<std::unordered_map<int32_t, pkv::Sequence>::node_type> spare;
  int32_t next_id = 0;
  // scratch of the batch calls, kept between calls so that a steady decode
  // loop allocates nothing on the host
  mutable uint64_t stamp = 0;
  mutable std::vector<pkv::Sequence*> batch;
  std::vector<int32_t> ref_delta;    // [num_blocks], all 0 between calls
  std::vector<int32_t> touched;      // blocks whose ref_delta is nonzero
};

namespace pkv {

void set_error(const std::string& msg);
pkv_status fail(pkv_status code, const std::string& msg);
int elem_bytes(int32_t dtype);

// Block references held outside sequence tables (the prefix cache): one more
// holder of block b; one fewer (back to the free queue at zero).
void block_ref(kv_pool* p, int32_t b);
void block_unref(kv_pool* p, int32_t b);
// A new sequence holding `blocks` (one more reference each) with `len`
// tokens; returns its id.  Caller checks ids are not exhausted.
int32_t adopt_sequence(kv_pool* p, const std::vector<int32_t>& blocks, int64_t len);

}  // namespace pkv
