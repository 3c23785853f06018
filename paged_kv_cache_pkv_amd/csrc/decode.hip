// Decode attention over the paged KV cache: split-K partials + merge pass.
//
// Each row's one query reads its keys and values in place through its block
// table (Build a continuous batching server, scalablesystem.dev,
// "PagedAttention Block Table Lookup") and attends over every cached
// position including the token appended this step (Inference
// Infrastructure, seeitflow.com, "Three iterations with the state written
// out").  The context is cut into fixed ranges of kSplitBlocks blocks; each
// range keeps the softmax statistics (running max m, running sum l,
// unnormalised output o) that let tiles combine exactly (The inference
// engine, wpnews.pro, "IO-aware attention and quantization attack different
// costs"), and a merge pass combines ranges.  A row that fits one range is
// written directly.  Ranges depend only on the row's own length, so a row's
// output is independent of its batch neighbours.
//
// Mapping onto gfx950.  One wave64 owns one (row, head, range).  A 16-token
// block of one head is 4 KiB of keys followed (128 KiB later) by 4 KiB of
// values, stored [token][128].  Lane l works on dims 8*(l%16) .. +7 of tokens
// l/16, l/16 + 4, l/16 + 8, l/16 + 12: every load instruction moves four
// whole 256-byte token rows (1 KiB contiguous per wave), straight into
// registers -- each lane consumes exactly what it loads, so no LDS staging is
// needed.  Loads carry the non-temporal cache policy.  Scores are dot products of FP16 pairs accumulated in fp32
// (v_dot2_f32_f16), summed over the 16 lanes of a token with DPP moves.  Each
// group of 16 lanes keeps its own online-softmax state over its four tokens
// of every block; the four groups merge once at the end of the range.  Blocks
// are software-pipelined two ahead so a wave keeps 24 KiB in flight.

#include "device_common.h"

namespace pkv {
namespace {

// Tunables (compile-time; the split size must stay fixed for a given build so
// that a row's result never depends on its batch neighbours).
#ifndef PKV_SPLIT_BLOCKS
#define PKV_SPLIT_BLOCKS 16
#endif
#ifndef PKV_PREFETCH
#define PKV_PREFETCH 2
#endif
#ifndef PKV_XCD_REMAP
#define PKV_XCD_REMAP 1
#endif
// Cache-policy bits of the K/V buffer loads: 2 = nt (streaming).  Keys and
// values are read once per step, and on gfx950 the non-temporal policy lifts
// the scattered-slab read rate from ~5.2 to ~6.5 TB/s.
#ifndef PKV_MIN_WAVES
#define PKV_MIN_WAVES 1
#endif
#ifndef PKV_KV_CPOL
#define PKV_KV_CPOL 2
#endif
#ifndef PKV_WAVES
#define PKV_WAVES 8
#endif

constexpr int kSplitBlocks = PKV_SPLIT_BLOCKS;  // blocks per split-K range
constexpr int kWavesPerGroup = PKV_WAVES;       // heads per workgroup
constexpr int kDecodeThreads = 64 * kWavesPerGroup;
constexpr int kDepth = PKV_PREFETCH + 1;        // tiles held in registers
constexpr int kXcds = 8;
static_assert(kSplitBlocks >= 1 && kSplitBlocks <= 64, "a range's block ids must fit one wave");

struct KVTile {
  uint4 k[4];
  uint4 v[4];
};

// Load one block's K and V rows for this lane through a buffer resource that
// spans the head's K tile up to the end of its V tile (vdelta bytes apart);
// the resource's range check turns any stray offset into a zero read.
__device__ __forceinline__ void load_tile(KVTile& t, const uint16_t* __restrict__ kslab, int vdelta, int lane_off) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kslab), 0, vdelta + kBlockSize * kHeadDim * 2, 0x00020000);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    t.k[i] = bitcast<uint4>(__builtin_amdgcn_raw_buffer_load_b128(rs, (lane_off + i * 4 * kHeadDim) * 2, 0, PKV_KV_CPOL));
#pragma unroll
  for (int i = 0; i < 4; ++i)
    t.v[i] = bitcast<uint4>(
        __builtin_amdgcn_raw_buffer_load_b128(rs, vdelta + (lane_off + i * 4 * kHeadDim) * 2, 0, PKV_KV_CPOL));
}

struct SoftmaxState {
  float m;
  float l;
  float o[8];
};

// Fold one block's four tokens (of this lane's group) into the state.
// valid = number of live tokens in the block (16 unless it is the last one).
__device__ __forceinline__ void fold_tile(SoftmaxState& st, KVTile& t, const uint4& q, float qk_scale, int group,
                                          int valid) {
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = sum16(dot8(q, t.k[i])) * qk_scale;
  if (valid < kBlockSize) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (group + 4 * i >= valid) {
        s[i] = -INFINITY;
        t.v[i] = make_uint4(0u, 0u, 0u, 0u);  // stale slots may hold NaN; 0 * NaN would leak
      }
    }
  }
  const float mb = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  const float mn = fmaxf(st.m, mb);
  const float alpha = fast_exp2(st.m - mn);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = fast_exp2(s[i] - mn);
  st.l = st.l * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack8(t.v[i], v[i]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc = st.o[e] * alpha;
    acc = fmaf(p[0], v[0][e], acc);
    acc = fmaf(p[1], v[1][e], acc);
    acc = fmaf(p[2], v[2][e], acc);
    acc = fmaf(p[3], v[3][e], acc);
    st.o[e] = acc;
  }
  st.m = mn;
}

// Merge the four 16-lane groups' states; every lane ends with the same bits.
__device__ __forceinline__ void merge_groups(SoftmaxState& st) {
  float M = fmaxf(st.m, shfl_xor(st.m, 16));
  M = fmaxf(M, shfl_xor(M, 32));
  const float f = fast_exp2(st.m - M);
  st.l *= f;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.o[e] *= f;
  st.l += shfl_xor(st.l, 16);
  st.l += shfl_xor(st.l, 32);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    st.o[e] += shfl_xor(st.o[e], 16);
    st.o[e] += shfl_xor(st.o[e], 32);
  }
  st.m = M;
}

struct DecodeArgs {
  const uint16_t* pool;
  const uint4* q;       // [R][H][16] chunks of 8 halves
  uint4* out;           // [R][H][16]
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;        // [R][H][S][128]
  float2* part_ml;      // [R][H][S]
  int layer, num_blocks, num_layers, num_heads;
  int bt_stride, num_rows, max_context_len, max_splits;
  float qk_scale;       // scale * log2(e)
};

__global__ __launch_bounds__(kDecodeThreads, PKV_MIN_WAVES) void decode_split_kernel(DecodeArgs a) {
  // 1-D grid over (row, range, head group).  Workgroups go to the XCDs
  // round-robin by index; with the remap, the head groups of one (row,
  // range) land on one XCD back to back, so they share its L2 and TLB for
  // the same block slabs.
  const int head_groups = (a.num_heads + kWavesPerGroup - 1) / kWavesPerGroup;
  const int n = blockIdx.x;
#if PKV_XCD_REMAP
  const int m = n / kXcds;
  const int hg = m % head_groups;
  const int rs = (n % kXcds) + kXcds * (m / head_groups);
#else
  const int hg = n % head_groups;
  const int rs = n / head_groups;
#endif
  const int split = rs % a.max_splits;
  const int r = rs / a.max_splits;
  if (r >= a.num_rows) return;
  const int h = hg * kWavesPerGroup + (threadIdx.x >> 6);
  if (h >= a.num_heads) return;
  const int lane = threadIdx.x & 63;
  const int group = lane >> 4;  // token within each 4-token stripe
  const int chunk = lane & 15;  // dims 8*chunk .. 8*chunk+7

  int L = a.context_lens[r];
  L = L > a.max_context_len ? a.max_context_len : L;
  const size_t rh = (size_t)r * a.num_heads + h;
  if (L < 1) {
    if (split == 0 && lane < 16) a.out[rh * 16 + chunk] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int nsplit = (nb + kSplitBlocks - 1) / kSplitBlocks;
  if (split >= nsplit) return;
  const int b0 = split * kSplitBlocks;
  const int b1 = min(nb, b0 + kSplitBlocks);

  // One vector load brings this range's block ids; readlane hands them out.
  const int32_t* row_table = a.block_tables + (size_t)r * a.bt_stride;
  const int my_id = (lane < b1 - b0) ? row_table[b0 + lane] : 0;

  const uint4 q = a.q[rh * 16 + chunk];
  const int lane_off = group * kHeadDim + chunk * 8;
  SoftmaxState st;
  st.m = kMinusBig;
  st.l = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.o[e] = 0.0f;

  auto block_id = [&](int j) {
    const int id = __builtin_amdgcn_readlane(my_id, j - b0);
    return id;
  };
  auto slab_k = [&](int id) { return a.pool + slab_offset(id, a.layer, 0, h, a.num_layers, a.num_heads); };
  const int vdelta = a.num_heads * kBlockSize * kHeadDim * 2;  // bytes from a head's K tile to its V tile

  // Software pipeline: block j + kDepth - 1 is loading while block j is folded.
  KVTile tile[kDepth];
  bool ok[kDepth];
  auto issue = [&](KVTile& t, bool& good, int j) {
    const int id = block_id(j);
    good = (unsigned)id < (unsigned)a.num_blocks;
    const int safe = good ? id : 0;
    load_tile(t, slab_k(safe), vdelta, lane_off);
  };
#pragma unroll
  for (int u = 0; u < kDepth - 1; ++u)
    if (b0 + u < b1) issue(tile[u], ok[u], b0 + u);
  for (int j = b0; j < b1; j += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int jj = j + u;
      constexpr int kAhead = kDepth - 1;
      if (jj + kAhead < b1) issue(tile[(u + kAhead) % kDepth], ok[(u + kAhead) % kDepth], jj + kAhead);
      if (jj < b1) {
        const int valid = ok[u] ? min(L - jj * kBlockSize, kBlockSize) : 0;
        fold_tile(st, tile[u], q, a.qk_scale, group, valid);
      }
    }
  }
  merge_groups(st);

  if (nsplit == 1) {
    if (lane < 16) {
      const float inv = 1.0f / st.l;
      uint4 o;
      o.x = pack_half2(st.o[0] * inv, st.o[1] * inv);
      o.y = pack_half2(st.o[2] * inv, st.o[3] * inv);
      o.z = pack_half2(st.o[4] * inv, st.o[5] * inv);
      o.w = pack_half2(st.o[6] * inv, st.o[7] * inv);
      a.out[rh * 16 + chunk] = o;
    }
  } else {
    const size_t slot = rh * a.max_splits + split;
    if (lane < 16) {
      float4* po = reinterpret_cast<float4*>(a.part_o + slot * kHeadDim + chunk * 8);
      po[0] = make_float4(st.o[0], st.o[1], st.o[2], st.o[3]);
      po[1] = make_float4(st.o[4], st.o[5], st.o[6], st.o[7]);
    }
    if (lane == 0) a.part_ml[slot] = make_float2(st.m, st.l);
  }
}

// Merge the ranges of every (row, head) that has more than one.  One wave per
// (row, head).  Lane s holds range s's statistics, so the maximum and the
// weights w_s = exp2(m_s - M) come from one parallel load and a wave
// reduction; lane l then owns dims 2l, 2l+1 and accumulates w_s * o_s over the
// ranges in index order (independent loads, unrolled), so the result does not
// depend on which range finished first.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__global__ __launch_bounds__(kDecodeThreads) void decode_merge_kernel(DecodeArgs a) {
  const int r = blockIdx.x;
  const int h = blockIdx.y * kWavesPerGroup + (threadIdx.x >> 6);
  if (h >= a.num_heads) return;
  const int lane = threadIdx.x & 63;
  int L = a.context_lens[r];
  L = L > a.max_context_len ? a.max_context_len : L;
  if (L < 1) return;
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int nsplit = (nb + kSplitBlocks - 1) / kSplitBlocks;
  if (nsplit <= 1) return;
  const size_t rh = (size_t)r * a.num_heads + h;
  const float2* ml = a.part_ml + rh * a.max_splits;
  const float2* po = reinterpret_cast<const float2*>(a.part_o + rh * a.max_splits * kHeadDim) + lane;

  float M = kMinusBig;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int s = s0 + lane;
    M = fmaxf(M, s < nsplit ? ml[s].x : kMinusBig);
  }
  M = wave_max(M);
  float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    const int s = s0 + lane;
    const float2 mine = s < nsplit ? ml[s] : make_float2(kMinusBig, 0.0f);
    const float w_mine = fast_exp2(mine.x - M);
    const int n = min(64, nsplit - s0);
    int j = 0;
    for (; j + 4 <= n; j += 4) {
      float2 p[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) p[u] = po[(size_t)(s0 + j + u) * (kHeadDim / 2)];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), j + u));
        o0 = fmaf(p[u].x, w, o0);
        o1 = fmaf(p[u].y, w, o1);
      }
    }
    for (; j < n; ++j) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), j));
      const float2 p = po[(size_t)(s0 + j) * (kHeadDim / 2)];
      o0 = fmaf(p.x, w, o0);
      o1 = fmaf(p.y, w, o1);
    }
    // l = sum_s l_s w_s over this chunk, added in index order
    for (int jj = 0; jj < n; ++jj) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), jj));
      const float ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.y), jj));
      l = fmaf(ls, w, l);
    }
  }
  const float inv = 1.0f / l;
  reinterpret_cast<uint32_t*>(a.out)[rh * 64 + lane] = pack_half2(o0 * inv, o1 * inv);
}

int max_splits_for(int32_t max_context_len) {
  const int nb = (max_context_len + kBlockSize - 1) / kBlockSize;
  return (nb + kSplitBlocks - 1) / kSplitBlocks;
}

}  // namespace
}  // namespace pkv

extern "C" int32_t pkv_split_tokens(void) { return pkv::kSplitBlocks * pkv::kBlockSize; }

extern "C" size_t pkv_decode_workspace_size(const pkv_cache* cache, int32_t num_rows, int32_t max_context_len) {
  using namespace pkv;
  if (!cache || num_rows < 1 || max_context_len < 1 || cache->num_heads < 1) return 0;
  const size_t s = (size_t)max_splits_for(max_context_len);
  const size_t n = (size_t)num_rows * cache->num_heads * s;
  return align256(n * kHeadDim * sizeof(float)) + align256(n * sizeof(float2));
}

extern "C" int pkv_decode_attention(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                    const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                                    int32_t num_rows, int32_t max_context_len, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (layer < 0 || layer >= cache->num_layers) return fail(PKV_ERR_INVALID_ARG, "layer out of range");
  if (num_rows < 1) return fail(PKV_ERR_INVALID_ARG, "num_rows must be >= 1");
  if (!out || !q || !block_tables || !context_lens) return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (bt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "bt_stride must be >= 1");
  if (max_context_len < 1 || (int64_t)max_context_len > (int64_t)bt_stride * kBlockSize)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len must be in [1, bt_stride * 16]");
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite and > 0");
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q) |
       reinterpret_cast<uintptr_t>(cache->base)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "out, q and cache->base must be 16-byte aligned");
  const int ms = max_splits_for(max_context_len);
  const size_t need = pkv_decode_workspace_size(cache, num_rows, max_context_len);
  if (ms > 1) {
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  DecodeArgs a;
  a.pool = static_cast<const uint16_t*>(cache->base);
  a.q = static_cast<const uint4*>(q);
  a.out = static_cast<uint4*>(out);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t n = (size_t)num_rows * cache->num_heads * ms;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = workspace ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + align256(n * kHeadDim * sizeof(float)))
                        : nullptr;
  a.layer = layer;
  a.num_blocks = cache->num_blocks;
  a.num_layers = cache->num_layers;
  a.num_heads = cache->num_heads;
  a.bt_stride = bt_stride;
  a.num_rows = num_rows;
  a.max_context_len = max_context_len;
  a.max_splits = ms;
  a.qk_scale = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int head_groups = (cache->num_heads + kWavesPerGroup - 1) / kWavesPerGroup;
  int64_t rs_total = (int64_t)num_rows * ms;
#if PKV_XCD_REMAP
  rs_total = (rs_total + kXcds - 1) / kXcds * kXcds;
#endif
  const int64_t wgs = rs_total * head_groups;
  if (wgs > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  decode_split_kernel<<<dim3((unsigned)wgs), dim3(kDecodeThreads), 0, s>>>(a);
  if (int rc = check_launch("decode split kernel")) return rc;
  if (ms > 1) {
    decode_merge_kernel<<<dim3(num_rows, head_groups), dim3(kDecodeThreads), 0, s>>>(a);
    if (int rc = check_launch("decode merge kernel")) return rc;
  }
  return PKV_OK;
}
