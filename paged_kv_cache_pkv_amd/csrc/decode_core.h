// Decode core shared by the decode launch, the mixed prefill launch and the
// shared-prefix suffix pass: a workgroup folds one (row, head, range of
// blocks) of a paged context with an online softmax, its waves taking equal
// shares of the range.  See decode.hip for the mapping onto gfx950.
#pragma once

#include "device_common.h"

namespace pkv {

// Tunables (compile-time; the split size must stay fixed for a given build so
// that a row's result never depends on its batch neighbours).
#ifndef PKV_SPLIT_BLOCKS
#define PKV_SPLIT_BLOCKS 16
#endif
// Cache-policy bits of the K/V buffer loads: 2 = nt (streaming).  Keys and
// values are read once per step, and on gfx950 the non-temporal policy lifts
// the scattered-slab read rate from ~5.2 to ~6.5 TB/s.
#ifndef PKV_KV_CPOL
#define PKV_KV_CPOL 2
#endif

// Waves that share one range, and the tiles each holds in registers while it
// folds its share (blocks in flight = depth - 1).
#ifndef PKV_RANGE_WAVES
#define PKV_RANGE_WAVES 4
#endif
#ifndef PKV_RANGE_DEPTH
#define PKV_RANGE_DEPTH 3
#endif

constexpr int kSplitBlocks = PKV_SPLIT_BLOCKS;  // blocks per split-K range
constexpr int kRangeWaves = PKV_RANGE_WAVES;
constexpr int kRangeDepth = PKV_RANGE_DEPTH;
static_assert(kSplitBlocks % kRangeWaves == 0, "each wave takes an equal share of a range");
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

// Fold one block's four tokens (of this lane's group) into the states of G
// queries that share the block's keys and values (the query heads of one KV
// head; G = 1 without grouping).  The values are unpacked once for all G.
// valid = number of live tokens in the block (16 unless it is the last one).
template <int G>
__device__ __forceinline__ void fold_tile(SoftmaxState* st, KVTile& t, const uint4* q, float qk_scale, int group,
                                          int valid) {
  float s[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) s[g][i] = sum16(dot8(q[g], t.k[i])) * qk_scale;
  if (valid < kBlockSize) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (group + 4 * i >= valid) {
#pragma unroll
        for (int g = 0; g < G; ++g) s[g][i] = -INFINITY;
        t.v[i] = make_uint4(0u, 0u, 0u, 0u);  // stale slots may hold NaN; 0 * NaN would leak
      }
    }
  }
  float p[G][4], alpha[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float mb = fmaxf(fmaxf(s[g][0], s[g][1]), fmaxf(s[g][2], s[g][3]));
    const float mn = fmaxf(st[g].m, mb);
    alpha[g] = fast_exp2(st[g].m - mn);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[g][i] = fast_exp2(s[g][i] - mn);
    st[g].l = st[g].l * alpha[g] + ((p[g][0] + p[g][1]) + (p[g][2] + p[g][3]));
    st[g].m = mn;
  }
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) unpack8(t.v[i], v[i]);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float acc = st[g].o[e] * alpha[g];
      acc = fmaf(p[g][0], v[0][e], acc);
      acc = fmaf(p[g][1], v[1][e], acc);
      acc = fmaf(p[g][2], v[2][e], acc);
      acc = fmaf(p[g][3], v[3][e], acc);
      st[g].o[e] = acc;
    }
}

// The same fold for G >= 2 query heads per KV head, where the vector work per
// byte grows with G.  Two changes keep it small:
//  - the exponent reference m moves only when a block's maximum passes it by
//    more than kGroupLazy (log2 units), so the common block rescales nothing
//    and its weights stay below 2^kGroupLazy;
//  - the weights are rounded to FP16 and P*V runs as v_dot2_f32_f16 over
//    pairs of tokens (one FP16 pair of values per dim), half the
//    instructions of fp32 multiply-adds on unpacked values.  The row sum adds
//    the same rounded weights, so numerator and denominator agree.
constexpr float kGroupLazy = 8.0f;

template <int G>
__device__ __forceinline__ void fold_tile_group(SoftmaxState* st, KVTile& t, const uint4* q, float qk_scale, int group,
                                                int valid) {
  float s[G][4];  // raw dot products; the scale is applied with the reference
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) s[g][i] = sum16(dot8(q[g], t.k[i]));
  if (valid < kBlockSize) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (group + 4 * i >= valid) {
#pragma unroll
        for (int g = 0; g < G; ++g) s[g][i] = -INFINITY;
        t.v[i] = make_uint4(0u, 0u, 0u, 0u);  // stale slots may hold NaN; 0 * NaN would leak
      }
    }
  }
  float mb[G];
  bool move = false;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mb[g] = fmaxf(fmaxf(s[g][0], s[g][1]), fmaxf(s[g][2], s[g][3])) * qk_scale;
    move = move || mb[g] > st[g].m + kGroupLazy;
  }
  if (__any(move)) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mn = fmaxf(st[g].m, mb[g]);
      const float alpha = fast_exp2(st[g].m - mn);
      st[g].l *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) st[g].o[e] *= alpha;
      st[g].m = mn;
    }
  }
  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
  half2_t p01[G], p23[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    p01[g].x = (_Float16)fast_exp2(fmaf(s[g][0], qk_scale, -st[g].m));
    p01[g].y = (_Float16)fast_exp2(fmaf(s[g][1], qk_scale, -st[g].m));
    p23[g].x = (_Float16)fast_exp2(fmaf(s[g][2], qk_scale, -st[g].m));
    p23[g].y = (_Float16)fast_exp2(fmaf(s[g][3], qk_scale, -st[g].m));
    st[g].l = __builtin_amdgcn_fdot2(p23[g], ones, __builtin_amdgcn_fdot2(p01[g], ones, st[g].l, false), false);
  }
  // values as FP16 pairs (token 4i, token 4i + 1 of this lane's stripe) per dim
  half2_t v01[8], v23[8];
  const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&t.v[0]);
  const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&t.v[1]);
  const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&t.v[2]);
  const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&t.v[3]);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const half2_t a = bitcast<half2_t>(w0[w]), b = bitcast<half2_t>(w1[w]);
    const half2_t c = bitcast<half2_t>(w2[w]), d = bitcast<half2_t>(w3[w]);
    v01[2 * w] = half2_t{a.x, b.x};
    v01[2 * w + 1] = half2_t{a.y, b.y};
    v23[2 * w] = half2_t{c.x, d.x};
    v23[2 * w + 1] = half2_t{c.y, d.y};
  }
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      st[g].o[e] = __builtin_amdgcn_fdot2(p23[g], v23[e], __builtin_amdgcn_fdot2(p01[g], v01[e], st[g].o[e], false),
                                          false);
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

// Fold blocks [b0, b1) (at most 64) of a context of L >= 1 tokens of KV head
// h_kv into the softmax states of its G query heads on one wave, then merge
// the four 16-lane groups so that every lane holds the same states.  q_head
// points at the first query head's 16 chunks (the G heads are consecutive,
// 16 chunks apart).  Depth = blocks whose loads are in flight per wave (plus
// the one being folded); the fold order, and so the result, does not depend
// on it.
//
// With new_k non-null, the context's last token (position L - 1, in block
// b1 - 1) is this step's new token: its keys and values come from new_k /
// new_v (16 chunks of this KV head) rather than from the pool, and the wave
// also writes them into their pool slot -- the append of that token for this
// head.  The bits folded are the ones an append followed by this fold would
// read back, so the result is the same.
template <int Depth, int G>
__device__ __forceinline__ void fold_blocks(const uint16_t* __restrict__ pool, int layer, int num_blocks,
                                            int num_layers, int num_kv_heads, int h_kv,
                                            const int32_t* __restrict__ row_table, int L, int b0, int b1,
                                            const uint4* __restrict__ q_head, float qk_scale, SoftmaxState* st,
                                            const uint4* __restrict__ new_k = nullptr,
                                            const uint4* __restrict__ new_v = nullptr) {
  const int lane = threadIdx.x & 63;
  const int group = lane >> 4;  // token within each 4-token stripe
  const int chunk = lane & 15;  // dims 8*chunk .. 8*chunk+7
  uint4 nk = make_uint4(0u, 0u, 0u, 0u), nv = nk;
  if (new_k) {
    nk = new_k[chunk];
    nv = new_v[chunk];
  }

  // One vector load brings the blocks' ids; readlane hands them out.
  const int my_id = (lane < b1 - b0) ? row_table[b0 + lane] : 0;
  uint4 q[G];
#pragma unroll
  for (int g = 0; g < G; ++g) q[g] = q_head[g * 16 + chunk];
  const int lane_off = group * kHeadDim + chunk * 8;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    st[g].m = kMinusBig;
    st[g].l = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st[g].o[e] = 0.0f;
  }

  const uint16_t* head_base = pool + slab_offset(0, layer, 0, h_kv, num_layers, num_kv_heads);
  const size_t block_stride = (size_t)num_layers * 2 * num_kv_heads * kBlockSize * kHeadDim;
  const int vdelta = num_kv_heads * kBlockSize * kHeadDim * 2;  // bytes from a head's K tile to its V tile

  // Software pipeline: block j + Depth - 1 is loading while block j is folded.
  KVTile tile[Depth];
  bool ok[Depth];
  auto issue = [&](KVTile& t, bool& good, int j) {
    const int id = __builtin_amdgcn_readlane(my_id, j - b0);
    good = (unsigned)id < (unsigned)num_blocks;
    const int safe = good ? id : 0;
    load_tile(t, head_base + (size_t)safe * block_stride, vdelta, lane_off);
  };
#pragma unroll
  for (int u = 0; u < Depth - 1; ++u)
    if (b0 + u < b1) issue(tile[u], ok[u], b0 + u);
  for (int j = b0; j < b1; j += Depth) {
#pragma unroll
    for (int u = 0; u < Depth; ++u) {
      const int jj = j + u;
      constexpr int kAhead = Depth - 1;
      if (jj + kAhead < b1) issue(tile[(u + kAhead) % Depth], ok[(u + kAhead) % Depth], jj + kAhead);
      if (jj < b1) {
        const int valid = ok[u] ? min(L - jj * kBlockSize, kBlockSize) : 0;
        if (new_k && jj == b1 - 1 && ok[u]) {
          // slot s of the last block holds the new token: lanes of group s % 4,
          // stripe entry s / 4
          const int s = (L - 1) & (kBlockSize - 1);
          const bool mine = group == (s & 3);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (mine && i == (s >> 2)) {
              tile[u].k[i] = nk;
              tile[u].v[i] = nv;
            }
          if (mine) {
            const int id = __builtin_amdgcn_readlane(my_id, jj - b0);
            uint16_t* slot_k = const_cast<uint16_t*>(head_base) + (size_t)id * block_stride + s * kHeadDim + chunk * 8;
            *reinterpret_cast<uint4*>(slot_k) = nk;
            *reinterpret_cast<uint4*>(reinterpret_cast<char*>(slot_k) + vdelta) = nv;
          }
        }
        if constexpr (G == 1)
          fold_tile<1>(st, tile[u], q, qk_scale, group, valid);
        else
          fold_tile_group<G>(st, tile[u], q, qk_scale, group, valid);
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) merge_groups(st[g]);
}

// LDS that the W waves of one range combine through (one per workgroup).
template <int W>
struct RangeScratchW {
  float4 o[W][32];  // each wave's unnormalised output, 128 floats
  float m[W];
  float l[W];
};
using RangeScratch = RangeScratchW<kRangeWaves>;

// Leave one wave's folded state in lds (lane l < 16 holds dims 8l .. 8l+7).
template <int W>
__device__ __forceinline__ void store_share(const SoftmaxState& st, RangeScratchW<W>& lds, int wave) {
  const int lane = threadIdx.x & 63;
  if (lane < 16) {
    lds.o[wave][2 * lane] = make_float4(st.o[0], st.o[1], st.o[2], st.o[3]);
    lds.o[wave][2 * lane + 1] = make_float4(st.o[4], st.o[5], st.o[6], st.o[7]);
  }
  if (lane == 0) {
    lds.m[wave] = st.m;
    lds.l[wave] = st.l;
  }
}

// One wave of a range's workgroup folds its share (see decode_range_waves)
// and leaves its softmax state in lds.
__device__ __forceinline__ void fold_range_share(const uint16_t* __restrict__ pool, int layer, int num_blocks,
                                                 int num_layers, int num_kv_heads, int h_kv,
                                                 const int32_t* __restrict__ row_table, int L, int b0, int b1,
                                                 const uint4* __restrict__ q_head, float qk_scale,
                                                 const uint4* __restrict__ new_k, const uint4* __restrict__ new_v,
                                                 RangeScratch& lds) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int kPer = kSplitBlocks / kRangeWaves;
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int w0 = min(b1, b0 + wave * kPer);
  const int w1 = min(b1, w0 + kPer);
  const bool takes_new = new_k != nullptr && w0 < w1 && w1 == nb;
  SoftmaxState st;
  fold_blocks<kRangeDepth, 1>(pool, layer, num_blocks, num_layers, num_kv_heads, h_kv, row_table, L, w0, w1, q_head,
                              qk_scale, &st, takes_new ? new_k : nullptr, takes_new ? new_v : nullptr);
  store_share(st, lds, wave);
}

// The same shares for nh query heads hq0 .. hq0 + nh - 1 (q_first is head
// hq0's query, the next heads' follow it), state of head j to lds[j], with no
// new token.  The tile loads run on across the heads' boundaries, so a wave
// waits for memory once rather than once per head; each head's blocks fold in
// the same order with the same arithmetic as in fold_range_share, so its state
// has the same bits.  q_per_kv query heads share a KV head.
template <int Depth>
__device__ __forceinline__ void fold_share_heads(const uint16_t* __restrict__ pool, int layer, int num_blocks,
                                                 int num_layers, int num_kv_heads, int q_per_kv, int hq0, int nh,
                                                 const int32_t* __restrict__ row_table, int L, int b0, int b1,
                                                 const uint4* __restrict__ q_first, float qk_scale,
                                                 RangeScratch* lds) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int group = lane >> 4;
  const int chunk = lane & 15;
  constexpr int kPer = kSplitBlocks / kRangeWaves;
  const int w0 = min(b1, b0 + wave * kPer);
  const int n = min(b1, w0 + kPer) - w0;  // blocks in this wave's share
  SoftmaxState st;
  auto reset = [&]() {
    st.m = kMinusBig;
    st.l = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.o[e] = 0.0f;
  };
  reset();
  if (n <= 0) {
    // an empty share: the state fold_blocks leaves for no blocks
    merge_groups(st);
    for (int j = 0; j < nh; ++j) store_share(st, lds[j], wave);
    return;
  }
  const int my_id = (lane < n) ? row_table[w0 + lane] : 0;
  const size_t block_stride = (size_t)num_layers * 2 * num_kv_heads * kBlockSize * kHeadDim;
  const int vdelta = num_kv_heads * kBlockSize * kHeadDim * 2;
  const int lane_off = group * kHeadDim + chunk * 8;
  auto head_base = [&](int j) {
    return pool + slab_offset(0, layer, 0, (hq0 + j) / q_per_kv, num_layers, num_kv_heads);
  };

  // issue cursor: item (ij, ik) = block w0 + ik of head ij
  int ij = 0, ik = 0;
  const uint16_t* ibase = head_base(0);
  KVTile tile[Depth];
  bool ok[Depth];
  auto issue = [&](KVTile& t, bool& good) {
    const int id = __builtin_amdgcn_readlane(my_id, ik);
    good = (unsigned)id < (unsigned)num_blocks;
    load_tile(t, ibase + (size_t)(good ? id : 0) * block_stride, vdelta, lane_off);
    if (++ik == n) {
      ik = 0;
      if (++ij < nh) ibase = head_base(ij);
    }
  };
  const int total = nh * n;
#pragma unroll
  for (int u = 0; u < Depth - 1; ++u)
    if (u < total) issue(tile[u], ok[u]);
  // the next head's query is loaded a head ahead (clamped to the last head,
  // so that the load needs no branch)
  uint4 q = q_first[chunk];
  uint4 q_next = q_first[min(1, nh - 1) * 16 + chunk];
  int fj = 0, fk = 0;  // fold cursor
  for (int i = 0; i < total; i += Depth) {
#pragma unroll
    for (int u = 0; u < Depth; ++u) {
      const int ii = i + u;
      constexpr int kAhead = Depth - 1;
      if (ii + kAhead < total) issue(tile[(u + kAhead) % Depth], ok[(u + kAhead) % Depth]);
      if (ii < total) {
        const int jj = w0 + fk;
        const int valid = ok[u] ? min(L - jj * kBlockSize, kBlockSize) : 0;
        fold_tile<1>(&st, tile[u], &q, qk_scale, group, valid);
        if (++fk == n) {
          merge_groups(st);
          store_share(st, lds[fj], wave);
          fk = 0;
          ++fj;
          reset();
          q = q_next;
          q_next = q_first[min(fj + 1, nh - 1) * 16 + chunk];
        }
      }
    }
  }
}

// One wave combines the range's shares from lds, in wave order, and writes
// the result: the normalised FP16 output when the row fits one range
// (single), otherwise the partial and its (m, l).  Lane l owns dims 2l, 2l+1;
// a share with no blocks holds m = kMinusBig and l = 0, so it adds nothing.
template <int W>
__device__ __forceinline__ void combine_range(const RangeScratchW<W>& lds, bool single,
                                              uint32_t* __restrict__ out_head, float* __restrict__ part_o,
                                              float2* __restrict__ part_ml) {
  const int lane = threadIdx.x & 63;
  float M = kMinusBig;
#pragma unroll
  for (int w = 0; w < W; ++w) M = fmaxf(M, lds.m[w]);
  float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const float f = fast_exp2(lds.m[w] - M);
    const float2 v = reinterpret_cast<const float2*>(&lds.o[w][0])[lane];
    l = fmaf(lds.l[w], f, l);
    o0 = fmaf(v.x, f, o0);
    o1 = fmaf(v.y, f, o1);
  }
  if (single) {
    const float inv = 1.0f / l;
    out_head[lane] = pack_half2(o0 * inv, o1 * inv);
  } else {
    reinterpret_cast<float2*>(part_o)[lane] = make_float2(o0, o1);
    if (lane == 0) *part_ml = make_float2(M, l);
  }
}

// Fold the blocks [b0, b1) of one row's range for one query head on a
// workgroup of kRangeWaves waves.  Wave w folds the w-th equal share of the
// range (kSplitBlocks / kRangeWaves blocks); the waves' softmax states then
// combine in wave order (The inference engine, wpnews.pro: the statistics of
// tiles combine exactly), so the result depends only on the range.  With
// single (the row fits one range) wave 0 writes the normalised FP16 output to
// out_head (64 pairs of halves); otherwise the unnormalised partial (128
// floats) to part_o and (m, l) to *part_ml.  With new_k / new_v, the wave
// whose share ends at the row's last block takes that token's keys and values
// and writes them into its slot (the fused append).  Every wave of the
// workgroup must call this: it synchronises the workgroup.
__device__ __forceinline__ void decode_range_waves(const uint16_t* __restrict__ pool, int layer, int num_blocks,
                                                   int num_layers, int num_kv_heads, int h_kv,
                                                   const int32_t* __restrict__ row_table, int L, int b0, int b1,
                                                   bool single, const uint4* __restrict__ q_head, float qk_scale,
                                                   const uint4* __restrict__ new_k, const uint4* __restrict__ new_v,
                                                   uint32_t* __restrict__ out_head, float* __restrict__ part_o,
                                                   float2* __restrict__ part_ml, RangeScratch& lds) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  fold_range_share(pool, layer, num_blocks, num_layers, num_kv_heads, h_kv, row_table, L, b0, b1, q_head, qk_scale,
                   new_k, new_v, lds);
  __syncthreads();
  if (wave == 0) combine_range(lds, single, out_head, part_o, part_ml);
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

// Up to PKV_MERGE_FAST_MAX ranges, every load of a merge goes out in one
// round trip (on the average mix 32 measured 0.5% faster per decode call
// than 8, with the same bits).
#ifndef PKV_MERGE_FAST
#define PKV_MERGE_FAST 1
#endif
#ifndef PKV_MERGE_FAST_MAX
#define PKV_MERGE_FAST_MAX 32
#endif

// merge_partials for nsplit <= N ranges, with all loads in one round trip.
template <int N>
__device__ __forceinline__ void merge_partials_one_trip(const float* __restrict__ part_o, const float2* __restrict__ ml,
                                                        int nsplit, uint32_t* __restrict__ out_head) {
  const int lane = threadIdx.x & 63;
  const float2* pf = reinterpret_cast<const float2*>(part_o) + lane;
  const float2 mine = lane < nsplit ? ml[lane] : make_float2(kMinusBig, 0.0f);
  float2 p[N];
#pragma unroll
  for (int u = 0; u < N; ++u) p[u] = u < nsplit ? pf[(size_t)u * (kHeadDim / 2)] : make_float2(0.0f, 0.0f);
  const float M = wave_max(mine.x);
  const float w_mine = fast_exp2(mine.x - M);
  float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    if (u < nsplit) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), u));
      o0 = fmaf(p[u].x, w, o0);
      o1 = fmaf(p[u].y, w, o1);
    }
  }
#pragma unroll
  for (int u = 0; u < N; ++u) {
    if (u < nsplit) {
      const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_mine), u));
      const float ls = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine.y), u));
      l = fmaf(ls, w, l);
    }
  }
  const float inv = 1.0f / l;
  out_head[lane] = pack_half2(o0 * inv, o1 * inv);
}

__device__ __forceinline__ void merge_partials(const float* __restrict__ part_o, const float2* __restrict__ ml,
                                               int nsplit, uint32_t* __restrict__ out_head) {
  const int lane = threadIdx.x & 63;
#if PKV_MERGE_FAST
  // Up to 8 (or 32) ranges: every statistic and partial load goes out in one
  // round trip (none depends on the maximum); the arithmetic is the general
  // path's, in the same order, so the bits are the same.
  if (nsplit <= 8) {
    merge_partials_one_trip<8>(part_o, ml, nsplit, out_head);
    return;
  }
  if (nsplit <= PKV_MERGE_FAST_MAX) {
    merge_partials_one_trip<PKV_MERGE_FAST_MAX>(part_o, ml, nsplit, out_head);
    return;
  }
#endif
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
