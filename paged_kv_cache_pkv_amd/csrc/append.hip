// KV append: scatter each new token's keys and values into its block slot.
//
// A decode step writes one key and one value vector per head for every new
// token into slot position % 16 of block block_table[position / 16]; a row
// takes a new block every 16 tokens and nothing is ever copied to grow it
// (LLM inference batching, faangrind, scheduler step 7; Build a continuous
// batching server, scalablesystem.dev, "PagedAttention Block Table Lookup":
// O(1) per appended token instead of a relayout).
//
// HBM-bound bit copy: 2 x heads x 256 B read and written per token.  One
// workgroup per token; each lane moves 16-byte chunks, so a wave writes
// four contiguous 256-byte head rows per instruction.

#include "device_common.h"

namespace pkv {
namespace {

constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void append_kernel(
    uint16_t* __restrict__ pool, int layer, int num_blocks, int num_layers, int num_heads,
    const uint4* __restrict__ k_new, const uint4* __restrict__ v_new, const int32_t* __restrict__ positions,
    const int32_t* __restrict__ request_of_token, const int32_t* __restrict__ block_tables, int num_rows,
    int bt_stride) {
  const int t = blockIdx.x;
  const int chunks = num_heads * (kHeadDim / 8);  // 16-byte chunks per K (or V) of one token
  // The token's data does not depend on where it goes: its loads are issued
  // first, so that they overlap the dependent reads of the row, the position
  // and the block id.
  constexpr int kPer = 4;  // chunks per lane in flight
  for (int c0 = 0; c0 < 2 * chunks; c0 += kPer * kAppendThreads) {
    uint4 val[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = c0 + u * kAppendThreads + threadIdx.x;
      const bool is_v = c >= chunks;
      val[u] = c < 2 * chunks ? (is_v ? v_new : k_new)[(size_t)t * chunks + (is_v ? c - chunks : c)]
                             : make_uint4(0u, 0u, 0u, 0u);
    }
    const int r = request_of_token[t];
    const int p = positions[t];
    if (r < 0 || r >= num_rows || p < 0 || (p >> 4) >= bt_stride) return;
    const int b = block_tables[(size_t)r * bt_stride + (p >> 4)];
    if (b < 0 || b >= num_blocks) return;
    const int slot = p & 15;
    const size_t k_slab = slab_offset(b, layer, 0, 0, num_layers, num_heads);
    const size_t v_slab = slab_offset(b, layer, 1, 0, num_layers, num_heads);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int c = c0 + u * kAppendThreads + threadIdx.x;
      if (c >= 2 * chunks) continue;
      const bool is_v = c >= chunks;
      const int rem = is_v ? c - chunks : c;
      const int h = rem >> 4;
      const int part = rem & 15;
      const size_t dst = (is_v ? v_slab : k_slab) + (size_t)h * (kBlockSize * kHeadDim) + slot * kHeadDim + part * 8;
      *reinterpret_cast<uint4*>(pool + dst) = val[u];
    }
  }
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_append(const pkv_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                          const int32_t* positions, const int32_t* request_of_token, int32_t num_tokens,
                          const int32_t* block_tables, int32_t num_rows, int32_t bt_stride, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (layer < 0 || layer >= cache->num_layers) return fail(PKV_ERR_INVALID_ARG, "layer out of range");
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) {
    clear_error();
    return PKV_OK;
  }
  if (!k_new || !v_new || !positions || !request_of_token || !block_tables)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (num_rows < 1 || bt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "num_rows and bt_stride must be >= 1");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
       reinterpret_cast<uintptr_t>(cache->base)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "k_new, v_new and cache->base must be 16-byte aligned");
  append_kernel<<<dim3(num_tokens), dim3(kAppendThreads), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<uint16_t*>(cache->base), layer, cache->num_blocks, cache->num_layers, cache->num_heads,
      static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), positions, request_of_token,
      block_tables, num_rows, bt_stride);
  return check_launch("pkv_append");
}
