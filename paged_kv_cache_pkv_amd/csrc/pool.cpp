// Host block pool: a stack-shaped free list plus one reference count per block.
//
// Allocation pops from the top and release pushes in the order given, as the
// block managers of Build a continuous batching server (scalablesystem.dev,
// "The KV Cache Block Manager (PagedAttention)") and Serving LLMs
// (sreshtalluri.github.io, "Paged KV memory") do; growth is all or nothing so
// a caller that comes up short can preempt someone instead.  Reference counts
// follow the faangrind data model's ref_count: a shared block goes back to the
// free list only when its last holder releases it.
//
// Every call checks all of its arguments before it changes any state.

#include <algorithm>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "pkv.h"
#include "pkv_internal.h"

struct pkv_pool {
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> refs;        // per block id
  std::vector<int32_t> scratch;     // per-call multiplicity counts, same size as refs
};

namespace {

bool ids_in_range(const pkv_pool* p, const int32_t* ids, int32_t n) {
  const int32_t nb = static_cast<int32_t>(p->refs.size());
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= nb) {
      pkv::set_error("block id " + std::to_string(ids[i]) + " outside [0, " + std::to_string(nb) + ")");
      return false;
    }
  }
  return true;
}

int create(int32_t num_blocks, const int32_t* free_ids, int32_t n_free, pkv_pool** out) {
  if (!out) return pkv::fail(PKV_ERR_INVALID_ARG, "out is null");
  *out = nullptr;
  if (num_blocks < 1) return pkv::fail(PKV_ERR_INVALID_ARG, "num_blocks must be >= 1");
  pkv_pool* p = new (std::nothrow) pkv_pool;
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARG, "out of host memory");
  // Every allocation the pool will ever make happens here: the free stack is
  // reserved at its largest size, so a later release never reallocates it.
  try {
    p->refs.assign(static_cast<size_t>(num_blocks), 0);
    p->scratch.assign(static_cast<size_t>(num_blocks), 0);
    p->free_stack.reserve(static_cast<size_t>(num_blocks));
  } catch (const std::bad_alloc&) {
    delete p;
    return pkv::fail(PKV_ERR_INVALID_ARG, "out of host memory");
  }
  if (free_ids == nullptr) {
    p->free_stack.resize(static_cast<size_t>(num_blocks));
    for (int32_t i = 0; i < num_blocks; ++i) p->free_stack[i] = i;
  } else {
    for (int32_t i = 0; i < n_free; ++i) {
      const int32_t b = free_ids[i];
      if (b < 0 || b >= num_blocks || p->scratch[b]) {
        delete p;
        return pkv::fail(PKV_ERR_BAD_BLOCK, "free list must hold distinct ids in [0, num_blocks)");
      }
      p->scratch[b] = 1;
    }
    p->free_stack.assign(free_ids, free_ids + n_free);
    for (int32_t b = 0; b < num_blocks; ++b) {
      p->refs[b] = p->scratch[b] ? 0 : 1;
      p->scratch[b] = 0;
    }
  }
  *out = p;
  pkv::clear_error();
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_pool_create(int32_t num_blocks, pkv_pool** out) { return create(num_blocks, nullptr, 0, out); }

int pkv_pool_create_from_list(int32_t num_blocks, const int32_t* free_ids, int32_t n_free, pkv_pool** out) {
  if (n_free < 0 || n_free > num_blocks) return pkv::fail(PKV_ERR_INVALID_ARG, "n_free must be in [0, num_blocks]");
  if (n_free > 0 && !free_ids) return pkv::fail(PKV_ERR_INVALID_ARG, "free_ids is null");
  static const int32_t kEmpty = 0;
  return create(num_blocks, n_free ? free_ids : &kEmpty, n_free, out);
}

void pkv_pool_destroy(pkv_pool* pool) { delete pool; }

int pkv_alloc(pkv_pool* p, int32_t n, int32_t* out_ids) {
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARG, "pool is null");
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && !out_ids) return pkv::fail(PKV_ERR_INVALID_ARG, "out_ids is null");
  if (static_cast<size_t>(n) > p->free_stack.size())
    return pkv::fail(PKV_ERR_OUT_OF_BLOCKS, "need " + std::to_string(n) + " blocks, " +
                                                std::to_string(p->free_stack.size()) + " free");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = p->free_stack.back();
    p->free_stack.pop_back();
    p->refs[b] = 1;
    out_ids[i] = b;
  }
  pkv::clear_error();
  return PKV_OK;
}

int pkv_ref(pkv_pool* p, const int32_t* ids, int32_t n) {
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARG, "pool is null");
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && !ids) return pkv::fail(PKV_ERR_INVALID_ARG, "ids is null");
  if (!ids_in_range(p, ids, n)) return PKV_ERR_BAD_BLOCK;
  for (int32_t i = 0; i < n; ++i)
    if (p->refs[ids[i]] == 0)
      return pkv::fail(PKV_ERR_DOUBLE_FREE, "block " + std::to_string(ids[i]) + " is free; cannot share it");
  for (int32_t i = 0; i < n; ++i) {
    if (p->refs[ids[i]] == INT32_MAX) return pkv::fail(PKV_ERR_INVALID_ARG, "reference count overflow");
  }
  for (int32_t i = 0; i < n; ++i) p->refs[ids[i]] += 1;
  pkv::clear_error();
  return PKV_OK;
}

int pkv_free(pkv_pool* p, const int32_t* ids, int32_t n) {
  if (!p) return pkv::fail(PKV_ERR_INVALID_ARG, "pool is null");
  if (n < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n > 0 && !ids) return pkv::fail(PKV_ERR_INVALID_ARG, "ids is null");
  if (!ids_in_range(p, ids, n)) return PKV_ERR_BAD_BLOCK;
  // multiplicity check: an id listed k times needs a count >= k
  int bad = -1;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    if (++p->scratch[b] > p->refs[b] && bad < 0) bad = b;
  }
  for (int32_t i = 0; i < n; ++i) p->scratch[ids[i]] = 0;
  if (bad >= 0)
    return pkv::fail(PKV_ERR_DOUBLE_FREE, "block " + std::to_string(bad) + " released more often than it is held");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    if (--p->refs[b] == 0) p->free_stack.push_back(b);
  }
  pkv::clear_error();
  return PKV_OK;
}

int pkv_grow(pkv_pool* p, int32_t* table, int32_t* table_len, int32_t capacity, int32_t num_tokens) {
  if (!p || !table_len) return pkv::fail(PKV_ERR_INVALID_ARG, "pool or table_len is null");
  if (num_tokens < 0 || capacity < 0 || *table_len < 0 || *table_len > capacity)
    return pkv::fail(PKV_ERR_INVALID_ARG, "need num_tokens >= 0 and 0 <= table_len <= capacity");
  const int32_t want = pkv_blocks_needed(num_tokens);
  const int32_t need = want - *table_len;
  if (need <= 0) {
    pkv::clear_error();
    return PKV_OK;
  }
  if (!table) return pkv::fail(PKV_ERR_INVALID_ARG, "table is null");
  if (want > capacity) return pkv::fail(PKV_ERR_INVALID_ARG, "table capacity too small");
  const int rc = pkv_alloc(p, need, table + *table_len);
  if (rc != PKV_OK) return rc;
  *table_len = want;
  return PKV_OK;
}

int pkv_grow_rows(pkv_pool* p, int32_t* tables, int32_t stride, int32_t* table_lens, const int32_t* num_tokens,
                  int32_t num_rows, int32_t* rows_grown) {
  if (!p || !rows_grown) return pkv::fail(PKV_ERR_INVALID_ARG, "pool or rows_grown is null");
  *rows_grown = 0;
  if (num_rows < 0 || stride < 1) return pkv::fail(PKV_ERR_INVALID_ARG, "need num_rows >= 0 and stride >= 1");
  if (num_rows > 0 && (!tables || !table_lens || !num_tokens))
    return pkv::fail(PKV_ERR_INVALID_ARG, "tables, table_lens or num_tokens is null");
  for (int32_t r = 0; r < num_rows; ++r) {
    if (num_tokens[r] < 0 || table_lens[r] < 0 || table_lens[r] > stride)
      return pkv::fail(PKV_ERR_INVALID_ARG, "row " + std::to_string(r) + ": need num_tokens >= 0 and 0 <= table_len <= stride");
    if (pkv_blocks_needed(num_tokens[r]) > stride)
      return pkv::fail(PKV_ERR_INVALID_ARG, "row " + std::to_string(r) + ": table stride too small");
  }
  for (int32_t r = 0; r < num_rows; ++r) {
    const int rc = pkv_grow(p, tables + static_cast<size_t>(r) * stride, table_lens + r, stride, num_tokens[r]);
    if (rc != PKV_OK) return rc;  // OUT_OF_BLOCKS: rows before r keep their growth
    *rows_grown = r + 1;
  }
  pkv::clear_error();
  return PKV_OK;
}

int32_t pkv_num_free(const pkv_pool* p) { return p ? static_cast<int32_t>(p->free_stack.size()) : -1; }

int32_t pkv_num_blocks(const pkv_pool* p) { return p ? static_cast<int32_t>(p->refs.size()) : -1; }

int32_t pkv_ref_count(const pkv_pool* p, int32_t id) {
  if (!p || id < 0 || id >= static_cast<int32_t>(p->refs.size())) return -1;
  return p->refs[id];
}

int32_t pkv_free_list(const pkv_pool* p, int32_t* out, int32_t cap) {
  if (!p) return -1;
  const int32_t n = static_cast<int32_t>(p->free_stack.size());
  if (out && cap > 0) std::memcpy(out, p->free_stack.data(), sizeof(int32_t) * static_cast<size_t>(std::min(n, cap)));
  return n;
}

int32_t pkv_blocks_needed(int32_t num_tokens) {
  if (num_tokens <= 0) return 0;
  return static_cast<int32_t>((static_cast<int64_t>(num_tokens) + 15) / 16);
}

}  // extern "C"
