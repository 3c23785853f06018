// Chunked-prefill attention on MFMA, mixed with decode rows in one launch.
//
// A prefill chunk's queries are the last n positions of its row's context;
// their keys and values were appended before the call and the chunk attends
// over its whole paged prefix plus itself under the causal rule (The
// inference engine, wpnews.pro, "Prefill and decode ask the accelerator for
// different work": large matrix operations that respect the causal mask).
// Chunks and decode rows share the step as one flat token list tagged by
// request (LLM inference batching, faangrind, "Prefill and decode share each
// step"), so one launch serves both.
//
// Prefill tiles (rows with n >= 2).  A workgroup of 4 waves owns 128 queries
// of one head and one fixed range of kPrefillSplit keys; wave w owns 32
// queries.  Keys advance 64 at a time (four 16-token blocks gathered through
// the block table) and are staged in LDS: K as [key][dim], V transposed as
// [dim][key] with the key order inside each group of 16 bit-swapped (bits 2
// and 3) so that the MFMA operand of P*V is one 16-byte LDS read.  On
// v_mfma_f32_32x32x16_f16:
//   S^T = K Q^T      A = K rows from LDS, B = the wave's queries (registers)
//   O^T += V^T P^T   A = V^T rows from LDS, B = P straight from S^T's registers
// In S^T's accumulator layout every query's 64 scores sit in two lanes
// (l and l ^ 32), so the softmax row maximum is one cross-lane exchange.  The
// online-softmax statistics combine across key steps and across ranges
// exactly (The inference engine, wpnews.pro, "IO-aware attention and
// quantization attack different costs").  Key ranges are fixed per row
// length, so a row's result does not depend on its batch neighbours.
//
// Decode rows (n == 1) in the same grid run the decode core (one wave per
// head and 256-token range).  A merge launch combines the ranges of every
// query that has more than one.

#include "decode_core.h"

namespace pkv {
namespace {

constexpr int kPrefillThreads = 256;
constexpr int kPrefillWaves = kPrefillThreads / 64;
constexpr int kQPerWave = 32;
constexpr int kBQ = kPrefillWaves * kQPerWave;  // queries per tile
constexpr int kBK = 64;                         // keys per step
#ifndef PKV_PREFILL_SPLIT
#define PKV_PREFILL_SPLIT 2048
#endif
constexpr int kPrefillSplit = PKV_PREFILL_SPLIT;  // keys per range
static_assert(kPrefillSplit % kBK == 0, "ranges hold whole key steps");
constexpr int kKRow = kHeadDim * 2 + 16;   // LDS bytes per K row (padded)
constexpr int kVRow = kBK * 2 + 16;        // LDS bytes per V^T row (padded)
constexpr int kKBytes = kBK * kKRow;
constexpr int kVBytes = kHeadDim * kVRow;
constexpr int kLdsBytes = kKBytes + kVBytes;
constexpr int kXcds = 8;

// V^T rows hold 8 chunks of 16 bytes (8 key positions each).  Chunk c of row d
// is stored at chunk c ^ ((d >> 3) & 7): the 16 rows a store instruction hits
// then fall in different banks instead of all in one (144-byte rows repeat
// every 8 rows modulo the bank count).
__device__ __forceinline__ int vt_offset(int d, int pos) {
  const int chunk = (pos >> 3) ^ ((d >> 3) & 7);
  return d * kVRow + chunk * 16 + (pos & 7) * 2;
}

struct PrefillArgs {
  const uint16_t* pool;
  const uint16_t* q;           // [T][H][128]
  uint16_t* out;               // [T][H][128]
  const int32_t* query_start;  // [R + 1]
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;               // [T][H][S][128]
  float2* part_ml;             // [T][H][S]
  int layer, num_blocks, num_layers, num_heads;
  int bt_stride, num_rows, total_q, max_context_len, max_splits;
  int tiles_max, ranges_max;   // prefill grid factors
  int prefill_wgs;             // workgroups [0, prefill_wgs) are prefill tiles (a multiple of kXcds)
  float qk_scale;              // scale * log2(e)
};

__device__ __forceinline__ int wave_prefix_sum(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __builtin_amdgcn_ds_bpermute(max(lane - off, 0) << 2, v);
    if (lane >= off) v += u;
  }
  return v;
}

__device__ __forceinline__ int row_queries(const int32_t* qs, int r) { return qs[r + 1] - qs[r]; }

// Map a global tile index onto (row, tile within the row) over rows with at
// least two queries; returns false past the last tile.
__device__ bool find_tile(const PrefillArgs& a, int tile, int& row, int& qtile) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int r0 = 0; r0 < a.num_rows; r0 += 64) {
    const int r = r0 + lane;
    int t = 0;
    if (r < a.num_rows) {
      const int n = row_queries(a.query_start, r);
      t = n >= 2 ? (n + kBQ - 1) / kBQ : 0;
    }
    const int incl = wave_prefix_sum(t) + base;
    const unsigned long long hit = __ballot(r < a.num_rows && tile < incl);
    if (hit) {
      const int first = __builtin_ctzll(hit);
      const int incl_first = __builtin_amdgcn_readlane(incl, first);
      const int t_first = __builtin_amdgcn_readlane(t, first);
      row = r0 + first;
      qtile = tile - (incl_first - t_first);
      return true;
    }
    base = __builtin_amdgcn_readlane(incl, 63);
  }
  return false;
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ h8 as_h8(const uint4& v) { return bitcast<h8>(v); }

__device__ void prefill_tile(const PrefillArgs& a, int r, int qtile, int h, int kr, char* __restrict__ lds) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int col = lane & 31;   // query column of this lane in the wave's 32
  const int half = lane >> 5;  // which 8 of each 16 reduction elements the lane holds
  const int qs0 = a.query_start[r];
  const int n = a.query_start[r + 1] - qs0;
  int L = a.context_lens[r];
  L = L > a.max_context_len ? a.max_context_len : L;
  if (L < n || qs0 < 0 || qs0 + n > a.total_q) return;  // contract violated: unspecified output, no access
  const int q_begin = qtile * kBQ;
  const int q_end = min(n, q_begin + kBQ);
  const int p_last = L - n + q_end - 1;  // last position in the tile
  const int k_begin = kr * kPrefillSplit;
  if (k_begin > p_last) return;  // no query of the tile reaches this range
  const int k_end = min(k_begin + kPrefillSplit, p_last + 1);

  const int wq = q_begin + wave * kQPerWave + col;  // this lane's query (row-local index)
  const bool q_ok = wq < q_end;
  const int p_q = q_ok ? L - n + wq : -1;
  const int wq0 = q_begin + wave * kQPerWave;  // the wave's first query
  const int p_wave_last = wq0 < q_end ? L - n + min(q_end, wq0 + kQPerWave) - 1 : -1;
  const int p_wave_first = L - n + wq0;

  // The wave's queries as MFMA B operands: Q[wq][16k + 8*half .. +7], k = 0..7.
  h8 qf[8];
  {
    const uint16_t* qrow = a.q + ((size_t)(qs0 + (q_ok ? wq : q_begin)) * a.num_heads + h) * kHeadDim + 8 * half;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint4 v = q_ok ? *reinterpret_cast<const uint4*>(qrow + 16 * k) : make_uint4(0u, 0u, 0u, 0u);
      qf[k] = as_h8(v);
    }
  }

  float16_t o[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.0f;
  float m = kMinusBig, lsum = 0.0f;

  const int32_t* row_table = a.block_tables + (size_t)r * a.bt_stride;
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const size_t block_stride = (size_t)a.num_layers * 2 * a.num_heads * kBlockSize * kHeadDim;
  const uint16_t* k_head = a.pool + slab_offset(0, a.layer, 0, h, a.num_layers, a.num_heads);
  const uint16_t* v_head = a.pool + slab_offset(0, a.layer, 1, h, a.num_layers, a.num_heads);

  // Per step each thread moves 4 K chunks (token tid/16 of each of the 4
  // blocks) and 4 V chunks (tokens 4*(tid/16 % 4) + j of block tid/64).
  uint4 kreg[4], vreg[4];
  const int ktok = tid >> 4, dchunk = tid & 15;
  const int kq = tid >> 4;  // key quad of the step for V: keys 4kq .. 4kq+3
  auto load_step = [&](int kb) {
    const int jb = kb / kBlockSize;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = jb + i;
      const int id = j < nb ? row_table[j] : -1;
      const bool ok = (unsigned)id < (unsigned)a.num_blocks && kb + 16 * i + ktok < L;
      kreg[i] = ok ? *reinterpret_cast<const uint4*>(k_head + (size_t)id * block_stride + ktok * kHeadDim + dchunk * 8)
                   : make_uint4(0u, 0u, 0u, 0u);
    }
    const int j = jb + (kq >> 2);
    const int id = j < nb ? row_table[j] : -1;
    const bool vid_ok = (unsigned)id < (unsigned)a.num_blocks;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int tok = 4 * (kq & 3) + t;
      const bool ok = vid_ok && kb + 4 * kq + t < L;
      vreg[t] = ok ? *reinterpret_cast<const uint4*>(v_head + (size_t)id * block_stride + tok * kHeadDim + dchunk * 8)
                   : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(lds + (16 * i + ktok) * kKRow + dchunk * 16) = kreg[i];
    // keys 4kq..4kq+3 sit in group kq/4 at positions 4 * swap(kq % 4) .. +3
    const int qi = kq & 3;
    const int pos = 16 * (kq >> 2) + 4 * (((qi & 1) << 1) | (qi >> 1));
    char* vt = lds + kKBytes;
    const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
    const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
    const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
    const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint2 pair;
      pair.x = __builtin_amdgcn_perm(w1[e >> 1], w0[e >> 1], sel);
      pair.y = __builtin_amdgcn_perm(w3[e >> 1], w2[e >> 1], sel);
      *reinterpret_cast<uint2*>(vt + vt_offset(dchunk * 8 + e, pos)) = pair;
    }
  };
  auto compute_step = [&](int kb) {
    float16_t s[2];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[T][i] = 0.0f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const h8 ka = *reinterpret_cast<const h8*>(lds + (32 * T + col) * kKRow + (16 * k + 8 * half) * 2);
        s[T] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[k], s[T], 0, 0, 0);
      }
    }
    // S^T[key = kb + 32T + 8(i/4) + 4*half + i%4][query col].  Keys past a
    // query's position only occur on the diagonal steps.
    if (kb + kBK - 1 > p_wave_first) {
#pragma unroll
      for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + 32 * T + 8 * (i >> 2) + 4 * half + (i & 3);
          if (key > p_q) s[T][i] = -INFINITY;
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, s[T][i]);
    mloc = fmaxf(mloc, shfl_xor(mloc, 32)) * a.qk_scale;  // scaled maximum of this step
    const float mn = fmaxf(m, mloc);
    if (__any(mn > m)) {  // the running maximum moved for some query: rescale
      const float alpha = fast_exp2(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
      m = mn;
    }
    float psum = 0.0f;
    h8 pb[4];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[T][i], a.qk_scale, -m));
        psum += p;
        pb[2 * T + (i >> 3)][i & 7] = (_Float16)p;
      }
    lsum += psum;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const h8 va = *reinterpret_cast<const h8*>(lds + kKBytes + vt_offset(32 * dt + col, 16 * kk + 8 * half));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[kk], o[dt], 0, 0, 0);
      }
  };

  load_step(k_begin);
  for (int kb = k_begin; kb < k_end; kb += kBK) {
    __syncthreads();  // the previous step's LDS reads are done
    store_step();
    __syncthreads();
    const bool more = kb + kBK < k_end;
    if (more) load_step(kb + kBK);  // next step's global loads fly during the MFMAs
    if (kb <= p_wave_last) compute_step(kb);
  }

  lsum += shfl_xor(lsum, 32);
  if (!q_ok) return;
  const int nsplit_q = p_q / kPrefillSplit + 1;
  if (kr >= nsplit_q) return;
  const size_t th = (size_t)(qs0 + wq) * a.num_heads + h;
  if (nsplit_q == 1) {
    const float inv = 1.0f / lsum;
    uint16_t* orow = a.out + th * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * half;
        uint2 w;
        w.x = pack_half2(o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv);
        w.y = pack_half2(o[dt][4 * g + 2] * inv, o[dt][4 * g + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
  } else {
    const size_t slot = th * a.max_splits + kr;
    float* po = a.part_o + slot * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dt + 8 * g + 4 * half;
        *reinterpret_cast<float4*>(po + d0) =
            make_float4(o[dt][4 * g], o[dt][4 * g + 1], o[dt][4 * g + 2], o[dt][4 * g + 3]);
      }
    if (half == 0) a.part_ml[slot] = make_float2(m, lsum);
  }
}

__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_mixed_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int n = blockIdx.x;
  if (n < a.prefill_wgs) {
    // XCD-aware order: consecutive logical indices run on one XCD, and the
    // innermost logical factor is the query tile, so the tiles that re-read
    // the same (head, key range) share that XCD's L2.
    const int per_xcd = a.prefill_wgs / kXcds;
    const int logical = (n % kXcds) * per_xcd + n / kXcds;
    const int tile = logical % a.tiles_max;
    const int rest = logical / a.tiles_max;
    const int kr = rest % a.ranges_max;
    const int h = rest / a.ranges_max;
    if (h >= a.num_heads) return;
    int row, qtile;
    if (!find_tile(a, tile, row, qtile)) return;
    prefill_tile(a, row, qtile, h, kr, lds);
    return;
  }
  // decode rows: (row, 256-token range, group of 4 heads)
  const int head_groups = (a.num_heads + kPrefillWaves - 1) / kPrefillWaves;
  const int d = n - a.prefill_wgs;
  const int hg = d % head_groups;
  const int rs = d / head_groups;
  const int split = rs % a.max_splits;
  const int r = rs / a.max_splits;
  if (r >= a.num_rows) return;
  const int h = hg * kPrefillWaves + (threadIdx.x >> 6);
  if (h >= a.num_heads) return;
  const int t = a.query_start[r];
  if (a.query_start[r + 1] - t != 1 || t < 0 || t >= a.total_q) return;
  int L = a.context_lens[r];
  L = L > a.max_context_len ? a.max_context_len : L;
  const size_t th = (size_t)t * a.num_heads + h;
  if (L < 1) {
    if (split == 0 && (threadIdx.x & 63) < 16)
      reinterpret_cast<uint4*>(a.out)[th * 16 + (threadIdx.x & 15)] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  if (split >= decode_splits(L)) return;
  const size_t slot = th * a.max_splits + split;
  decode_range(a.pool, a.layer, a.num_blocks, a.num_layers, a.num_heads, h, a.block_tables + (size_t)r * a.bt_stride, L,
               split, reinterpret_cast<const uint4*>(a.q) + th * 16, a.qk_scale,
               reinterpret_cast<uint4*>(a.out) + th * 16, a.part_o + slot * kHeadDim, a.part_ml + slot);
}

// One wave per (query token, head): find the token's row, count its ranges,
// merge when there is more than one.
__global__ __launch_bounds__(kPrefillThreads) void prefill_merge_kernel(PrefillArgs a) {
  const int t = blockIdx.x;
  const int h = blockIdx.y * kPrefillWaves + (threadIdx.x >> 6);
  if (h >= a.num_heads) return;
  int lo = 0, hi = a.num_rows - 1;  // last row with query_start[row] <= t
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.query_start[mid] <= t) lo = mid; else hi = mid - 1;
  }
  const int r = lo;
  const int qs0 = a.query_start[r];
  const int n = a.query_start[r + 1] - qs0;
  if (t - qs0 >= n) return;
  int L = a.context_lens[r];
  L = L > a.max_context_len ? a.max_context_len : L;
  if (L < 1 || L < n) return;
  int nsplit;
  if (n == 1) {
    nsplit = decode_splits(L);
  } else {
    const int p = L - n + (t - qs0);
    nsplit = p / kPrefillSplit + 1;
  }
  if (nsplit <= 1) return;
  const size_t th = (size_t)t * a.num_heads + h;
  merge_partials(a.part_o + th * a.max_splits * kHeadDim, a.part_ml + th * a.max_splits, nsplit,
                 reinterpret_cast<uint32_t*>(a.out) + th * 64);
}

int prefill_max_splits(int32_t max_context_len) {
  const int dec = decode_splits(max_context_len);
  const int pre = (max_context_len + kPrefillSplit - 1) / kPrefillSplit;
  return dec > pre ? dec : pre;
}

}  // namespace
}  // namespace pkv

extern "C" size_t pkv_prefill_workspace_size(const pkv_cache* cache, int32_t num_rows, int32_t total_q,
                                             int32_t max_q_per_row, int32_t max_context_len) {
  using namespace pkv;
  (void)num_rows;
  (void)max_q_per_row;
  if (!cache || total_q < 1 || max_context_len < 1 || cache->num_heads < 1) return 0;
  const size_t n = (size_t)total_q * cache->num_heads * prefill_max_splits(max_context_len);
  return align256(n * kHeadDim * sizeof(float)) + align256(n * sizeof(float2));
}

extern "C" int pkv_chunked_prefill_attention(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                             const int32_t* query_start, const int32_t* block_tables,
                                             int32_t bt_stride, const int32_t* context_lens, int32_t num_rows,
                                             int32_t total_q, int32_t max_q_per_row, int32_t max_context_len,
                                             float scale, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (layer < 0 || layer >= cache->num_layers) return fail(PKV_ERR_INVALID_ARG, "layer out of range");
  if (num_rows < 1 || total_q < 1) return fail(PKV_ERR_INVALID_ARG, "num_rows and total_q must be >= 1");
  if (!out || !q || !query_start || !block_tables || !context_lens)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (bt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "bt_stride must be >= 1");
  if (max_context_len < 1 || (int64_t)max_context_len > (int64_t)bt_stride * kBlockSize)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len must be in [1, bt_stride * 16]");
  if (max_q_per_row < 1 || max_q_per_row > max_context_len || max_q_per_row > total_q)
    return fail(PKV_ERR_INVALID_ARG, "max_q_per_row must be in [1, min(total_q, max_context_len)]");
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite and > 0");
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q) |
       reinterpret_cast<uintptr_t>(cache->base)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "out, q and cache->base must be 16-byte aligned");
  const size_t need = pkv_prefill_workspace_size(cache, num_rows, total_q, max_q_per_row, max_context_len);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");

  PrefillArgs a;
  a.pool = static_cast<const uint16_t*>(cache->base);
  a.q = static_cast<const uint16_t*>(q);
  a.out = static_cast<uint16_t*>(out);
  a.query_start = query_start;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.max_splits = prefill_max_splits(max_context_len);
  const size_t n = (size_t)total_q * cache->num_heads * a.max_splits;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + align256(n * kHeadDim * sizeof(float)));
  a.layer = layer;
  a.num_blocks = cache->num_blocks;
  a.num_layers = cache->num_layers;
  a.num_heads = cache->num_heads;
  a.bt_stride = bt_stride;
  a.num_rows = num_rows;
  a.total_q = total_q;
  a.max_context_len = max_context_len;
  a.qk_scale = scale * kLog2e;
  // Tiles: every row with n >= 2 wastes at most one partial tile, and rows
  // with n == 1 add none, so ceil(total_q / kBQ) + num_rows bounds the count.
  const int64_t tiles = max_q_per_row >= 2 ? ((int64_t)total_q + kBQ - 1) / kBQ + num_rows : 0;
  const int64_t ranges = ((int64_t)max_context_len + kPrefillSplit - 1) / kPrefillSplit;
  int64_t pre = tiles * ranges * cache->num_heads;
  pre = (pre + kXcds - 1) / kXcds * kXcds;
  const int head_groups = (cache->num_heads + kPrefillWaves - 1) / kPrefillWaves;
  const int64_t dec = (int64_t)num_rows * decode_splits(max_context_len) * head_groups;
  if (pre + dec > INT32_MAX || tiles > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  a.tiles_max = (int)(tiles > 0 ? tiles : 1);
  a.ranges_max = (int)ranges;
  a.prefill_wgs = (int)pre;
  hipStream_t s = static_cast<hipStream_t>(stream);
  prefill_mixed_kernel<<<dim3((unsigned)(pre + dec)), dim3(kPrefillThreads), 0, s>>>(a);
  if (int rc = check_launch("prefill mixed kernel")) return rc;
  prefill_merge_kernel<<<dim3((unsigned)total_q, (unsigned)head_groups), dim3(kPrefillThreads), 0, s>>>(a);
  return check_launch("prefill merge kernel");
}
