// Whole-block copies: copy-on-write inside the pool, and swap between the
// pool and host memory.
//
// Requests that share prefix blocks hold them immutable; when one branch
// diverges inside a shared block it gets a private copy of that block first
// (The inference engine, wpnews.pro, "Weights, activations, and KV state
// occupy different ledgers" and "Paging turns variable sequences into block
// tables": copy-on-write restores separate ownership).  When the pool runs
// out, a scheduler may move a sequence's blocks to host memory and restore
// them later instead of recomputing its prefill (Build a continuous batching
// server, scalablesystem.dev, "Preemption and Eviction: Recompute vs Swap";
// Inference Infrastructure, seeitflow.com, "An overload example").
//
// In the pool layout [block][layer][2][head][16][128] every block, all layers
// included, is one contiguous region of num_layers x 2 x heads x 4 KiB
// (8 MiB for 32 layers x 32 heads).  The copy kernel streams whole blocks
// with 16-byte non-temporal buffer loads and stores (HBM-bound: each byte is
// read once and written once); a swap is one DMA copy per run of
// consecutive block ids.

#include "device_common.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kCopyThreads = 256;
constexpr int kCopyChunk = 32 * 1024;  // bytes per workgroup

// grid.x = pair, grid.y = 32 KiB chunk of the block.  Pairs with an id
// outside the pool are skipped.
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(char* __restrict__ pool, size_t block_bytes,
                                                                   int num_blocks, const int32_t* __restrict__ src_ids,
                                                                   const int32_t* __restrict__ dst_ids) {
  const int src = src_ids[blockIdx.x];
  const int dst = dst_ids[blockIdx.x];
  if ((unsigned)src >= (unsigned)num_blocks || (unsigned)dst >= (unsigned)num_blocks) return;
  const size_t begin = (size_t)blockIdx.y * kCopyChunk;
  const int bytes = (int)min((size_t)kCopyChunk, block_bytes - begin);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(pool + (size_t)src * block_bytes + begin, 0, bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc(pool + (size_t)dst * block_bytes + begin, 0, bytes, 0x00020000);
  constexpr int kPer = kCopyChunk / (16 * kCopyThreads);  // 16-byte words per thread
  u32x4 v[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int off = (i * kCopyThreads + (int)threadIdx.x) * 16;
    v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2);  // reads past `bytes` return zero
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int off = (i * kCopyThreads + (int)threadIdx.x) * 16;
    __builtin_amdgcn_raw_buffer_store_b128(v[i], rd, off, 0, 2);  // writes past `bytes` are dropped
  }
}

size_t block_bytes_of(const pkv_cache* c) {
  return (size_t)c->num_layers * 2 * c->num_heads * kBlockSize * kHeadDim * sizeof(uint16_t);
}

// Host-side ids for a swap: all must be in range before anything is queued.
int check_host_ids(const pkv_cache* cache, const int32_t* ids, int32_t n) {
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= cache->num_blocks)
      return fail(PKV_ERR_BAD_BLOCK, "block id " + std::to_string(ids[i]) + " at index " + std::to_string(i) +
                                         " is outside the pool");
  return PKV_OK;
}

// One DMA copy per maximal run of consecutive ids (ids[i+1] == ids[i] + 1).
template <typename F>
int for_each_run(const int32_t* ids, int32_t n, F&& f) {
  int32_t i = 0;
  while (i < n) {
    int32_t j = i + 1;
    while (j < n && ids[j] == ids[j - 1] + 1) ++j;
    if (int rc = f(i, ids[i], j - i)) return rc;
    i = j;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" size_t pkv_block_bytes(const pkv_cache* cache) {
  using namespace pkv;
  if (check_cache(cache)) return 0;
  clear_error();
  return block_bytes_of(cache);
}

extern "C" int pkv_copy_blocks(const pkv_cache* cache, const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                               void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) {
    clear_error();
    return PKV_OK;
  }
  if (!src_ids || !dst_ids) return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (reinterpret_cast<uintptr_t>(cache->base) & 15) return fail(PKV_ERR_INVALID_ARG, "cache->base must be 16-byte aligned");
  const size_t bb = block_bytes_of(cache);
  const size_t chunks = (bb + kCopyChunk - 1) / kCopyChunk;
  if (chunks > 65535) return fail(PKV_ERR_UNSUPPORTED, "block larger than 2 GiB");
  copy_blocks_kernel<<<dim3((unsigned)n, (unsigned)chunks), dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<char*>(cache->base), bb, cache->num_blocks, src_ids, dst_ids);
  return check_launch("pkv_copy_blocks");
}

extern "C" int pkv_swap_out(const pkv_cache* cache, const int32_t* ids, int32_t n, void* host_dst, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) {
    clear_error();
    return PKV_OK;
  }
  if (!ids || !host_dst) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (int rc = check_host_ids(cache, ids, n)) return rc;
  const size_t bb = block_bytes_of(cache);
  const char* base = static_cast<const char*>(cache->base);
  char* host = static_cast<char*>(host_dst);
  const int rc = for_each_run(ids, n, [&](int32_t at, int32_t first, int32_t count) {
    const hipError_t e = hipMemcpyAsync(host + (size_t)at * bb, base + (size_t)first * bb, (size_t)count * bb,
                                        hipMemcpyDeviceToHost, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : fail(PKV_ERR_HIP, std::string("pkv_swap_out: ") + hipGetErrorString(e));
  });
  if (rc) return rc;
  clear_error();
  return PKV_OK;
}

extern "C" int pkv_swap_in(const pkv_cache* cache, const void* host_src, const int32_t* ids, int32_t n, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) {
    clear_error();
    return PKV_OK;
  }
  if (!ids || !host_src) return fail(PKV_ERR_INVALID_ARG, "null pointer");
  if (int rc = check_host_ids(cache, ids, n)) return rc;
  const size_t bb = block_bytes_of(cache);
  char* base = static_cast<char*>(cache->base);
  const char* host = static_cast<const char*>(host_src);
  const int rc = for_each_run(ids, n, [&](int32_t at, int32_t first, int32_t count) {
    const hipError_t e = hipMemcpyAsync(base + (size_t)first * bb, host + (size_t)at * bb, (size_t)count * bb,
                                        hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PKV_OK : fail(PKV_ERR_HIP, std::string("pkv_swap_in: ") + hipGetErrorString(e));
  });
  if (rc) return rc;
  clear_error();
  return PKV_OK;
}
