// Decode core shared by the decode launch and the mixed prefill launch: one
// wave folds one (row, head, range of blocks) of a paged context with an
// online softmax.  See decode.hip for the mapping onto gfx950.
#pragma once

#include "device_common.h"

namespace pkv {

// Tunables (compile-time; the split size must stay fixed for a given build so
// that a row's result never depends on its batch neighbours).
#ifndef PKV_SPLIT_BLOCKS
#define PKV_SPLIT_BLOCKS 16
#endif
#ifndef PKV_PREFETCH
#define PKV_PREFETCH 2
#endif
// Cache-policy bits of the K/V buffer loads: 2 = nt (streaming).  Keys and
// values are read once per step, and on gfx950 the non-temporal policy lifts
// the scattered-slab read rate from ~5.2 to ~6.5 TB/s.
#ifndef PKV_KV_CPOL
#define PKV_KV_CPOL 2
#endif

constexpr int kSplitBlocks = PKV_SPLIT_BLOCKS;  // blocks per split-K range
constexpr int kDepth = PKV_PREFETCH + 1;        // tiles held in registers
static_assert(kSplitBlocks >= 1 && kSplitBlocks <= 64, "a range's block ids must fit one wave");

__host__ __device__ constexpr int decode_splits(int L) {
  return ((L + kBlockSize - 1) / kBlockSize + kSplitBlocks - 1) / kSplitBlocks;
}

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

// Fold range `split` (blocks [split*kSplitBlocks, ...) of a context of L >= 1
// tokens) for head h on one wave.  With a single range for the row the
// normalised FP16 output goes to out_head (16 chunks of 8 halves); otherwise the
// unnormalised partial goes to part_o (128 floats) and (m, l) to *part_ml.
__device__ __forceinline__ void decode_range(const uint16_t* __restrict__ pool, int layer, int num_blocks,
                                             int num_layers, int num_heads, int h,
                                             const int32_t* __restrict__ row_table, int L, int split,
                                             const uint4* __restrict__ q_head, float qk_scale,
                                             uint4* __restrict__ out_head, float* __restrict__ part_o,
                                             float2* __restrict__ part_ml) {
  const int lane = threadIdx.x & 63;
  const int group = lane >> 4;  // token within each 4-token stripe
  const int chunk = lane & 15;  // dims 8*chunk .. 8*chunk+7
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int nsplit = (nb + kSplitBlocks - 1) / kSplitBlocks;
  const int b0 = split * kSplitBlocks;
  const int b1 = min(nb, b0 + kSplitBlocks);

  // One vector load brings this range's block ids; readlane hands them out.
  const int my_id = (lane < b1 - b0) ? row_table[b0 + lane] : 0;
  const uint4 q = q_head[chunk];
  const int lane_off = group * kHeadDim + chunk * 8;
  SoftmaxState st;
  st.m = kMinusBig;
  st.l = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.o[e] = 0.0f;

  const uint16_t* head_base = pool + slab_offset(0, layer, 0, h, num_layers, num_heads);
  const size_t block_stride = (size_t)num_layers * 2 * num_heads * kBlockSize * kHeadDim;
  const int vdelta = num_heads * kBlockSize * kHeadDim * 2;  // bytes from a head's K tile to its V tile

  // Software pipeline: block j + kDepth - 1 is loading while block j is folded.
  KVTile tile[kDepth];
  bool ok[kDepth];
  auto issue = [&](KVTile& t, bool& good, int j) {
    const int id = __builtin_amdgcn_readlane(my_id, j - b0);
    good = (unsigned)id < (unsigned)num_blocks;
    const int safe = good ? id : 0;
    load_tile(t, head_base + (size_t)safe * block_stride, vdelta, lane_off);
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
        fold_tile(st, tile[u], q, qk_scale, group, valid);
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
      out_head[chunk] = o;
    }
  } else {
    if (lane < 16) {
      float4* po = reinterpret_cast<float4*>(part_o + chunk * 8);
      po[0] = make_float4(st.o[0], st.o[1], st.o[2], st.o[3]);
      po[1] = make_float4(st.o[4], st.o[5], st.o[6], st.o[7]);
    }
    if (lane == 0) *part_ml = make_float2(st.m, st.l);
  }
}

// Merge `nsplit` > 1 partials of one (query, head) on one wave: lane s holds
// range s's statistics, so the maximum and the weights w_s = exp2(m_s - M)
// come from one parallel load and a wave reduction; lane l then owns dims
// 2l, 2l+1 and accumulates w_s * o_s over ranges in index order (independent
// loads, unrolled), so the result never depends on which range finished first.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}

__device__ __forceinline__ void merge_partials(const float* __restrict__ part_o, const float2* __restrict__ ml,
                                               int nsplit, uint32_t* __restrict__ out_head) {
  const int lane = threadIdx.x & 63;
  const float2* po = reinterpret_cast<const float2*>(part_o) + lane;
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
    // up to 16 independent partial loads in flight per lane
    for (; j + 16 <= n; j += 16) {
      float2 p[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) p[u] = po[(size_t)(s0 + j + u) * (kHeadDim / 2)];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), j + u));
        o0 = fmaf(p[u].x, w, o0);
        o1 = fmaf(p[u].y, w, o1);
      }
    }
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
    for (int jj = 0; jj < n; ++jj) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), jj));
      const float ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.y), jj));
      l = fmaf(ls, w, l);
    }
  }
  const float inv = 1.0f / l;
  out_head[lane] = pack_half2(o0 * inv, o1 * inv);
}

}  // namespace pkv
