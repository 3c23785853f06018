// Shared-prefix decode: when many rows of a decode step begin with the same
// reference-counted prefix blocks, read those blocks once per step for all of
// them.
//
// Prefix blocks are computed once, marked immutable and shared by reference
// count by every sequence whose prompt starts with them, so in a multi-tenant
// step the one shared prefix is read by every concurrent sequence (Build a
// continuous batching server, scalablesystem.dev, "Scaling and Performance";
// Serving LLMs, "Prefix caching": a 2,000-token system prompt stored once).
// The result is still every row's attention over its own context; only the
// reads change.  A row flagged as sharing a prefix of P blocks has its range
// partition cut at block P:
//   prefix ranges   blocks [16 s, min(16 s + 16, P)), s < ceil(P / 16)
//   own ranges      blocks [P + 16 k, ...) up to the row's last block
// and every range's partial softmax statistics combine exactly in the merge
// (The inference engine, wpnews.pro: tile statistics combine exactly).
//
// Three launches:
//   prefix_tile_kernel    one wave per (head, prefix range, 32 sharing rows):
//                         the 32 rows' decode queries form an MFMA tile, so
//                         the range's K and V cross HBM once per 32 rows
//                         instead of once per row;
//   prefix_suffix_kernel  the decode core over each row's own ranges (and the
//                         whole context of rows that share nothing);
//   prefix_merge_kernel   the decode merge over each row's ranges in order.
// The partition depends only on a row's length, its flag and P, so a row's
// output does not depend on its batch neighbours.

#include "decode_core.h"

namespace pkv {
namespace {

constexpr int kPxQ = 32;                              // sharing rows per prefix tile (one wave)
constexpr int kPxRowBytes = kHeadDim * 2;             // one key's 128 dims
constexpr int kPxBlockBytes = kBlockSize * kPxRowBytes;  // 4 KiB: one block of one head, K or V
constexpr int kPxStepBytes = 2 * kPxBlockBytes;       // a step is two blocks: 32 keys
constexpr int kPxXcds = 8;
constexpr int kSuffixWaves = 8;                       // heads per merge workgroup
constexpr int kSuffixThreads = 64 * kSuffixWaves;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
#define PKV_PX_LDS __attribute__((address_space(3)))

struct PrefixArgs {
  const uint16_t* pool;
  const uint4* q;              // [R][H][16 chunks of 8 halves]
  uint4* out;                  // [R][H][16]
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* shares;       // [R] nonzero: the row's first P table entries are the prefix's blocks
  float* part_o;               // [R][H][S][128]
  float2* part_ml;             // [R][H][S]
  int layer, num_blocks, num_layers, num_heads;
  int bt_stride, num_rows, max_context_len, max_splits;
  int prefix_blocks;           // P
  int prefix_ranges;           // ceil(P / kSplitBlocks)
  int tiles;                   // prefix tiles per (head, prefix range): ceil(R / 32)
  float qk_scale;              // scale * log2(e)
};

__device__ __forceinline__ int clamp_len(const PrefixArgs& a, int r) {
  const int L = a.context_lens[r];
  return L > a.max_context_len ? a.max_context_len : L;
}

// A flagged row takes the shared path only when its context runs past the
// prefix (its own new token always lies beyond the shared, immutable blocks);
// otherwise it is decoded like any other row.
__device__ __forceinline__ bool row_shares(const PrefixArgs& a, int L, int flag) {
  return a.prefix_blocks > 0 && flag != 0 && L > a.prefix_blocks * kBlockSize;
}

__device__ __forceinline__ int row_splits(const PrefixArgs& a, int L, bool shared) {
  if (!shared) return decode_splits(L);
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  return a.prefix_ranges + (nb - a.prefix_blocks + kSplitBlocks - 1) / kSplitBlocks;
}

__device__ __forceinline__ int px_wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __builtin_amdgcn_ds_bpermute(((lane - d) & 63) << 2, v);
    if (lane >= d) v += u;
  }
  return v;
}

// Position of 16-byte chunk c of LDS row r (rows of 256 bytes): swapping the
// two 2-bit halves of r & 15 spreads 16 consecutive rows, and the 4 rows x 4
// chunks of one transposed read, over distinct bank groups.
__device__ __forceinline__ int px_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

template <typename T>
__device__ __forceinline__ T* px_uniform(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

__shared__ __attribute__((aligned(16))) char g_px_k0[kPxStepBytes];
__shared__ __attribute__((aligned(16))) char g_px_k1[kPxStepBytes];
__shared__ __attribute__((aligned(16))) char g_px_v0[kPxStepBytes];
__shared__ __attribute__((aligned(16))) char g_px_v1[kPxStepBytes];
__shared__ int g_px_rows[kPxQ];

// One wave: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_f16 for
// 32 sharing rows' queries of head h over prefix range s, two blocks (32
// keys) per step, K and V double-buffered in LDS by direct global->LDS loads.
// Lane (col, half): query col; register i of S^T holds key 8(i/4) + 4 half +
// i%4 of the step, and register i of O^T tile dt holds dim 32 dt + 8(i/4) +
// 4 half + i%4.
__global__ __launch_bounds__(64) void prefix_tile_kernel(PrefixArgs a) {
  const int n = blockIdx.x;
  const int mq = n / kPxXcds;
  // the tiles of one (head, range) run back to back on one XCD and share its L2
  const int tile = mq % a.tiles;
  const int task = (n % kPxXcds) + kPxXcds * (mq / a.tiles);
  if (task >= a.num_heads * a.prefix_ranges) return;
  const int h = __builtin_amdgcn_readfirstlane(task % a.num_heads);
  const int s = __builtin_amdgcn_readfirstlane(task / a.num_heads);
  const int lane = threadIdx.x & 63;
  const int col = lane & 31;
  const int half = lane >> 5;

  // The tile's rows: the sharing rows of rank 32 tile .. 32 tile + 31, in row order.
  if (lane < kPxQ) g_px_rows[lane] = -1;
  __syncthreads();
  int count = 0;
  for (int r0 = 0; r0 < a.num_rows; r0 += 64) {
    const int r = r0 + lane;
    int f = 0;
    if (r < a.num_rows) f = row_shares(a, clamp_len(a, r), a.shares[r]) ? 1 : 0;
    const int rank = count + px_wave_inclusive_sum(f) - 1;
    if (f && rank >= kPxQ * tile && rank < kPxQ * (tile + 1)) g_px_rows[rank - kPxQ * tile] = r;
    count = __builtin_amdgcn_readlane(rank, 63) + 1;
    if (count >= kPxQ * (tile + 1)) break;
  }
  __syncthreads();
  if (count <= kPxQ * tile) return;  // fewer sharing rows than this tile's first rank
  const int row = g_px_rows[col];
  const int row0 = __builtin_amdgcn_readfirstlane(g_px_rows[0]);

  const int blk0 = s * kSplitBlocks;
  const int nblk = __builtin_amdgcn_readfirstlane(min(kSplitBlocks, a.prefix_blocks - blk0));
  const int nsteps = (nblk + 1) / 2;
  // the prefix's block ids come from the first row's table: every sharing
  // row's table begins with the same P ids
  const int32_t* table0 = a.block_tables + (size_t)row0 * a.bt_stride;
  const int ids = lane < nblk ? table0[blk0 + lane] : -1;

  const size_t block_stride = (size_t)a.num_layers * 2 * a.num_heads * kBlockSize * kHeadDim;
  const size_t vdelta = (size_t)a.num_heads * kBlockSize * kHeadDim;
  const uint16_t* head0 = a.pool + slab_offset(0, a.layer, 0, h, a.num_layers, a.num_heads);
  int voff[4];
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const int r = 4 * qd + (lane >> 4);
    voff[qd] = r * kPxRowBytes + (((lane & 15) ^ px_swz(r)) << 4);
  }
  // Block j of the range (two per step) into slot b of a step's K and V
  // buffers; a missing or invalid block reads as zeros (a buffer of zero
  // records) and its keys are masked below.
  auto issue = [&](char* kb, char* vb, int step) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int j = 2 * step + b;
      const int id = j < nblk ? __builtin_amdgcn_readlane(ids, j) : -1;
      const bool ok = (unsigned)id < (unsigned)a.num_blocks;
      const uint16_t* kbase = px_uniform(head0 + (ok ? (size_t)id * block_stride : 0));
      const int nrec = ok ? kPxBlockBytes : 0;
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase), 0, nrec, 0x00020000);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(kbase + vdelta), 0, nrec, 0x00020000);
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (PKV_PX_LDS void*)(kb + b * kPxBlockBytes + 4 * qd * kPxRowBytes), 16,
                                                 voff[qd], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (PKV_PX_LDS void*)(vb + b * kPxBlockBytes + 4 * qd * kPxRowBytes), 16,
                                                 voff[qd], 0, 0, 0);
      }
    }
  };
  auto block_ok = [&](int j) {
    const int id = j < nblk ? __builtin_amdgcn_readlane(ids, j) : -1;
    return (unsigned)id < (unsigned)a.num_blocks;
  };

  // The queries as MFMA B operands: Q[row][16 k + 8 half .. +7], k = 0..7.
  h8 qf[8];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) +
                           ((size_t)(row >= 0 ? row : row0) * a.num_heads + h) * kHeadDim + 8 * half;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 v = row >= 0 ? *reinterpret_cast<const uint4*>(qrow + 16 * k) : make_uint4(0u, 0u, 0u, 0u);
      qf[k] = bitcast<h8>(v);
    }
  }

  // Transposed V reads: in each 16-lane group g, source lane sl points at key
  // 8 rr + 4 (g >> 1) + sl / 4 and dims 32 dt + 16 (g & 1) + 4 (sl & 3) .. +3;
  // the read hands lane i of the group the 4 keys of dim 32 dt + 16 (g & 1) + i,
  // in the key order P has in S^T's registers.
  const int g = lane >> 4, sl = lane & 15;
  int v_byte[2][4];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int vr = 8 * rr + 4 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = 32 * dt + 16 * (g & 1) + 4 * (sl & 3);
      v_byte[rr][dt] = vr * kPxRowBytes + (((d >> 3) ^ px_swz(vr)) << 4) + (d & 7) * 2;
    }
  }

  float16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
  float m = kMinusBig, lsum = 0.0f;
  const float16_t zero = {};
  // The exponent reference m moves only when a score passes it by more than
  // kLazy (log2 units): weights stay below 2^kLazy, well inside FP16, and O
  // and the row sum are always relative to the same m.
  constexpr float kLazy = 8.0f;

  auto compute = [&](const char* kt, const char* vt, int step) {
    float16_t sc;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const h8 ka = *reinterpret_cast<const h8*>(kt + col * kPxRowBytes + (((2 * k + half) ^ px_swz(col)) << 4));
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[k], k == 0 ? zero : sc, 0, 0, 0);
    }
    // keys of a missing or invalid block get -inf (registers 0..7: the step's
    // first block, 8..15: its second)
    if (!block_ok(2 * step)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sc[i] = -INFINITY;
    }
    if (!block_ok(2 * step + 1)) {
#pragma unroll
      for (int i = 8; i < 16; ++i) sc[i] = -INFINITY;
    }
    float x = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) x = fmaxf(x, sc[i]);
    const auto both = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    const float mstep = fmaxf(__uint_as_float(both[0]), __uint_as_float(both[1])) * a.qk_scale;
    // Decided per query (both lanes of a query see the same mstep), so a
    // row's result never depends on the other rows of its tile.  A query
    // that keeps its reference scales by exactly 1.
    const float mn = mstep > m + kLazy ? mstep : m;
    if (__any(mn != m)) {
      const float alpha = fast_exp2(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      m = mn;
    }
    // weights rounded to FP16 as the P*V operand; the row sum adds the same FP16 values
    h8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) pb[i >> 3][i & 7] = (_Float16)fast_exp2(fmaf(sc[i], a.qk_scale, -m));
    const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};
    float ls = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const half2_t pair = {pb[kk][e], pb[kk][e + 1]};
        ls = __builtin_amdgcn_fdot2(pair, ones, ls, false);
      }
    lsum += ls;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const char* vb = vt + kk * kPxBlockBytes;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_PX_LDS v4i16*)(vb + v_byte[0][dt]));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_PX_LDS v4i16*)(vb + v_byte[1][dt]));
        const h8 va = bitcast<h8>(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[kk], o[dt], 0, 0, 0);
      }
  };

  // Step i uses buffers i % 2.  Each iteration waits for every load issued so
  // far (its own step) and for its previous LDS reads, refills the other
  // buffers with step i + 1, then computes step i.
  issue(g_px_k0, g_px_v0, 0);
  for (int i = 0; i < nsteps; i += 2) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    if (i + 1 < nsteps) issue(g_px_k1, g_px_v1, i + 1);
    compute(g_px_k0, g_px_v0, i);
    if (i + 1 >= nsteps) break;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    if (i + 2 < nsteps) issue(g_px_k0, g_px_v0, i + 2);
    compute(g_px_k1, g_px_v1, i + 1);
  }

  {
    const auto both = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(both[0]) + __uint_as_float(both[1]);
  }
  if (row < 0) return;
  const size_t slot = ((size_t)row * a.num_heads + h) * a.max_splits + s;
  float* po = a.part_o + slot * kHeadDim;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = 32 * dt + 8 * gq + 4 * half;
      *reinterpret_cast<float4*>(po + d0) =
          make_float4(o[dt][4 * gq], o[dt][4 * gq + 1], o[dt][4 * gq + 2], o[dt][4 * gq + 3]);
    }
  if (half == 0) a.part_ml[slot] = make_float2(m, lsum);
}

// The decode core over every range that is not a prefix range: a sharing
// row's own ranges from block P on, and the whole context of every other row.
// One workgroup per (row, range, head), its waves sharing the range as in the
// decode launch, so an unmarked row gets the decode launch's bits.
__global__ __launch_bounds__(64 * kRangeWaves) void prefix_suffix_kernel(PrefixArgs a) {
  __shared__ RangeScratch lds;
  const int n = blockIdx.x;
  const int mq = n / kPxXcds;
  const int h = mq % a.num_heads;
  const int rs = (n % kPxXcds) + kPxXcds * (mq / a.num_heads);
  const int split = rs % a.max_splits;
  const int r = rs / a.max_splits;
  if (r >= a.num_rows) return;
  const int L = clamp_len(a, r);
  const size_t rh = (size_t)r * a.num_heads + h;
  if (L < 1) {
    if (split == 0 && threadIdx.x < 16) a.out[rh * 16 + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const bool shared = row_shares(a, L, a.shares[r]);
  const int nsplit = row_splits(a, L, shared);
  if (split >= nsplit) return;
  int b0;
  if (shared) {
    if (split < a.prefix_ranges) return;  // folded by the prefix tiles
    b0 = a.prefix_blocks + (split - a.prefix_ranges) * kSplitBlocks;
  } else {
    b0 = split * kSplitBlocks;
  }
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int b1 = min(nb, b0 + kSplitBlocks);
  const size_t slot = rh * a.max_splits + split;
  decode_range_waves(a.pool, a.layer, a.num_blocks, a.num_layers, a.num_heads, h,
                     a.block_tables + (size_t)r * a.bt_stride, L, b0, b1, nsplit == 1, a.q + rh * 16, a.qk_scale,
                     nullptr, nullptr, reinterpret_cast<uint32_t*>(a.out) + rh * 64, a.part_o + slot * kHeadDim,
                     a.part_ml + slot, lds);
}

__global__ __launch_bounds__(kSuffixThreads) void prefix_merge_kernel(PrefixArgs a) {
  const int r = blockIdx.x;
  const int h = __builtin_amdgcn_readfirstlane(blockIdx.y * kSuffixWaves + (threadIdx.x >> 6));
  if (h >= a.num_heads) return;
  const int L = clamp_len(a, r);
  if (L < 1) return;
  const int nsplit = row_splits(a, L, row_shares(a, L, a.shares[r]));
  if (nsplit <= 1) return;
  const size_t rh = (size_t)r * a.num_heads + h;
  merge_partials(a.part_o + rh * a.max_splits * kHeadDim, a.part_ml + rh * a.max_splits, nsplit,
                 reinterpret_cast<uint32_t*>(a.out) + rh * 64);
}

int prefix_ranges_of(int32_t prefix_blocks) { return (prefix_blocks + kSplitBlocks - 1) / kSplitBlocks; }

}  // namespace
}  // namespace pkv

extern "C" size_t pkv_decode_workspace_size_prefix(const pkv_cache* cache, int32_t num_rows, int32_t max_context_len,
                                                   int32_t prefix_blocks) {
  using namespace pkv;
  if (!cache || num_rows < 1 || max_context_len < 1 || cache->num_heads < 1 || prefix_blocks < 0) return 0;
  const size_t s = (size_t)prefix_ranges_of(prefix_blocks) + decode_splits(max_context_len);
  const size_t n = (size_t)num_rows * cache->num_heads * s;
  return align256(n * kHeadDim * sizeof(float)) + align256(n * sizeof(float2));
}

extern "C" int pkv_decode_attention_prefix(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                           const int32_t* block_tables, int32_t bt_stride,
                                           const int32_t* context_lens, int32_t num_rows, int32_t max_context_len,
                                           float scale, const int32_t* shares_prefix, int32_t prefix_blocks,
                                           void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (layer < 0 || layer >= cache->num_layers) return fail(PKV_ERR_INVALID_ARG, "layer out of range");
  if (num_rows < 1) return fail(PKV_ERR_INVALID_ARG, "num_rows must be >= 1");
  if (!out || !q || !block_tables || !context_lens) return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (bt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "bt_stride must be >= 1");
  if (max_context_len < 1 || (int64_t)max_context_len > (int64_t)bt_stride * kBlockSize)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len must be in [1, bt_stride * 16]");
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (prefix_blocks < 0 || prefix_blocks > bt_stride)
    return fail(PKV_ERR_INVALID_ARG, "prefix_blocks must be in [0, bt_stride]");
  if (prefix_blocks > 0 && !shares_prefix) return fail(PKV_ERR_INVALID_ARG, "shares_prefix is null");
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "out and q must be 16-byte aligned");
  const int np = prefix_ranges_of(prefix_blocks);
  const int ms = np + decode_splits(max_context_len);
  const size_t need = pkv_decode_workspace_size_prefix(cache, num_rows, max_context_len, prefix_blocks);
  if (ms > 1) {
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  PrefixArgs a;
  a.pool = static_cast<const uint16_t*>(cache->base);
  a.q = static_cast<const uint4*>(q);
  a.out = static_cast<uint4*>(out);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.shares = prefix_blocks > 0 ? shares_prefix : context_lens;  // never read as flags when P = 0
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
  a.prefix_blocks = prefix_blocks;
  a.prefix_ranges = np;
  a.tiles = (num_rows + kPxQ - 1) / kPxQ;
  a.qk_scale = scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (np > 0) {
    const int64_t tasks = ((int64_t)cache->num_heads * np + kPxXcds - 1) / kPxXcds * kPxXcds;
    const int64_t wgs = tasks * a.tiles;
    if (wgs > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
    prefix_tile_kernel<<<dim3((unsigned)wgs), dim3(64), 0, st>>>(a);
    if (int rc = check_launch("prefix tile kernel")) return rc;
  }
  const int head_groups = (cache->num_heads + kSuffixWaves - 1) / kSuffixWaves;  // of the merge launch
  const int64_t rs_total = ((int64_t)num_rows * ms + kPxXcds - 1) / kPxXcds * kPxXcds;
  const int64_t wgs = rs_total * cache->num_heads;
  if (wgs > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  prefix_suffix_kernel<<<dim3((unsigned)wgs), dim3(64 * kRangeWaves), 0, st>>>(a);
  if (int rc = check_launch("prefix suffix kernel")) return rc;
  if (ms > 1) {
    prefix_merge_kernel<<<dim3(num_rows, head_groups), dim3(kSuffixThreads), 0, st>>>(a);
    if (int rc = check_launch("prefix merge kernel")) return rc;
  }
  return PKV_OK;
}
