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
// queries.  Keys advance 64 at a time: four 16-token blocks gathered through
// the block table by direct global->LDS loads (no registers), with K one step
// further ahead than V, so that each wave starts the next step's QK^T on the
// matrix cores before it computes this step's softmax on the vector ALUs.  K
// and V sit in LDS row-major; V reaches the MFMA transposed through
// ds_read_b64_tr_b16.  On v_mfma_f32_32x32x16_f16:
//   S^T = K Q^T      A = K rows from LDS, B = the wave's queries (registers)
//   O^T += V^T P^T   A = V^T via transposed LDS reads, B = P straight from
//                    S^T's registers
// In S^T's accumulator layout every query's 64 scores sit in two lanes
// (l and l ^ 32), so the softmax row maximum is one cross-lane exchange.  The
// online-softmax statistics combine across key steps and across ranges
// exactly (The inference engine, wpnews.pro, "IO-aware attention and
// quantization attack different costs").  Key ranges are fixed per row
// length, so a row's result does not depend on its batch neighbours.
//
// Decode rows (n == 1) in the same grid run the decode core (one workgroup
// per 256-token range and group of 4 heads, each head's range folded as in
// the decode launch).  A merge launch combines the ranges of every query that
// has more than one.

#include <type_traits>

#include "decode_core.h"

namespace pkv {
namespace {

constexpr int kPrefillThreads = 256;
constexpr int kPrefillWaves = kPrefillThreads / 64;
constexpr int kQPerWave = 32;
constexpr int kBQ = kPrefillWaves * kQPerWave;  // queries per tile
constexpr int kBK = 64;                         // keys per step
// Order of the mixed launch: -1 lets the host decide per call (see the
// launch), 0 puts every prefill tile first, 1 spreads the tiles among the
// decode workgroups.
#ifndef PKV_PREFILL_INTERLEAVE
#define PKV_PREFILL_INTERLEAVE -1
#endif
#ifndef PKV_PREFILL_SPLIT
#define PKV_PREFILL_SPLIT 2048
#endif
constexpr int kPrefillSplit = PKV_PREFILL_SPLIT;  // keys per range
static_assert(kPrefillSplit % kBK == 0, "ranges hold whole key steps");
static_assert(kPrefillSplit / kBK <= 64, "a range's block ids for one slot fit one wave");
constexpr int kRowBytes = kHeadDim * 2;        // one key's 128 dims
constexpr int kTileBytes = kBK * kRowBytes;     // K (or V) of one step: 16 KiB
constexpr int kXcds = 8;
// Tiles a decode wave of the mixed launch holds in registers (blocks in
// flight = depth - 1).
#ifndef PKV_MIXED_DEPTH
#define PKV_MIXED_DEPTH 4
#endif
static_assert(kPrefillWaves == 4, "one wave per block of a step");
static_assert(kPrefillWaves == kRangeWaves, "a decode workgroup of the mixed launch is one range's waves");
static_assert(kPrefillWaves * sizeof(RangeScratch) <= kTileBytes, "the decode waves combine in one K tile");

// LDS: three K tiles and two V tiles (80 KiB), as distinct objects so that
// the compiler can tell a tile being filled by direct loads from one being
// read.  Step i's keys sit in K tile i % 3 and its values in V tile i % 2:
// while step i's softmax and P*V run, the QK^T of step i+1 already reads its
// K tile.  Rows are 256 bytes (16 chunks of 16 bytes, no padding); chunk c of
// tile row r is stored at position c ^ swz(r), swz swapping the two 2-bit
// halves of r & 15.  Then the 16 consecutive rows of one K operand read land
// on 16 distinct positions, and so do the 4 rows x 4 chunks of one
// transposed V read: both are free of bank conflicts.
__shared__ __attribute__((aligned(16))) char g_k_tile0[kTileBytes];
__shared__ __attribute__((aligned(16))) char g_k_tile1[kTileBytes];
__shared__ __attribute__((aligned(16))) char g_k_tile2[kTileBytes];
__shared__ __attribute__((aligned(16))) char g_v_tile0[kTileBytes];
__shared__ __attribute__((aligned(16))) char g_v_tile1[kTileBytes];

template <int S>
__device__ __forceinline__ char* k_tile() {
  return S == 0 ? g_k_tile0 : S == 1 ? g_k_tile1 : g_k_tile2;
}
template <int S>
__device__ __forceinline__ char* v_tile() {
  return S == 0 ? g_v_tile0 : g_v_tile1;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
#define PKV_LDS __attribute__((address_space(3)))

struct PrefillArgs {
  const uint16_t* pool;
  const uint16_t* q;           // [T][H][128]
  uint16_t* out;               // [T][H][128]
  const int32_t* query_start;  // [R + 1]
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;               // [T][H][S][128]
  float2* part_ml;             // [T][H][S]
  int32_t* tok_splits;         // [T] ranges each query token was cut into
  int layer, num_blocks, num_layers, num_heads;  // num_heads: KV heads of the pool
  int num_q_heads, group;      // query heads; query head h reads KV head h / group
  int bt_stride, num_rows, total_q, max_context_len, max_splits;
  int tiles_max, ranges_max;   // prefill grid factors
  int prefill_wgs;             // prefill tile workgroups (a multiple of kXcds)
  int decode_wgs;              // decode workgroups (a multiple of kXcds)
  int interleave;              // spread the prefill tiles among the decode workgroups
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

__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

struct TileCtx {
  int ids;                  // lane i: block id of step i for this wave's block slot (or -1)
  const uint16_t* k_head;   // K tile of head h in block 0 of the layer
  size_t block_stride;      // elements between blocks
  size_t vdelta;            // elements from a head's K tile to its V tile
  int nb, L, num_blocks;
  int voff[4];              // this lane's source byte offsets for the 4 row quads of a block
};

// Each step gathers four 16-token blocks (kb / 16 + w, w = 0..3): wave w
// loads block w's K rows into a K tile or its V rows into a V tile, 4 direct
// 1 KiB global->LDS transfers in which each lane fetches the chunk that the
// swizzle puts in its LDS slot.  The buffer resource covers only the block's
// live rows, so rows past the context (and whole blocks with an invalid id)
// read as zero.
__device__ __forceinline__ void issue_rows(const TileCtx& c, char* tile, int kb, int step, bool is_v) {
  const int blk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int first = kb + kBlockSize * blk;
  int rows = c.L - first;
  rows = rows < 0 ? 0 : (rows > kBlockSize ? kBlockSize : rows);
  const int id = __builtin_amdgcn_readlane(c.ids, step);
  const bool ok = (unsigned)id < (unsigned)c.num_blocks && rows > 0;
  // block id and row count are wave-uniform; keep the resource words scalar
  const uint16_t* base =
      uniform_ptr(c.k_head + (ok ? (size_t)id * c.block_stride : 0) + (is_v ? c.vdelta : 0));
  const int nrec = __builtin_amdgcn_readfirstlane(ok ? rows * kRowBytes : 0);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, nrec, 0x00020000);
  char* dst = tile + kBlockSize * blk * kRowBytes;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (PKV_LDS void*)(dst + 4 * q * kRowBytes), 16, c.voff[q], 0, 0, 0);
}

// All of this wave's direct loads have landed and its LDS reads have
// returned; then the workgroup meets.
__device__ __forceinline__ void loads_barrier() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ void prefill_tile(const PrefillArgs& a, int r_in, int qtile_in, int h_in, int kr_in) {
  // the tile coordinates are workgroup-uniform; say so, so that block ids and
  // buffer resources stay in scalar registers
  const int r = __builtin_amdgcn_readfirstlane(r_in);
  const int qtile = __builtin_amdgcn_readfirstlane(qtile_in);
  const int h = __builtin_amdgcn_readfirstlane(h_in);
  const int kr = __builtin_amdgcn_readfirstlane(kr_in);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int p_wave_first = L - n + wq0;

  TileCtx c;
  {
    // one load brings every step's block id for this wave's block slot
    const int32_t* row_table = a.block_tables + (size_t)r * a.bt_stride;
    const int nb = (L + kBlockSize - 1) / kBlockSize;
    const int j = k_begin / kBlockSize + 4 * lane + wave;
    c.ids = (lane < kPrefillSplit / kBK && j < nb) ? row_table[j] : -1;
  }
  c.block_stride = (size_t)a.num_layers * 2 * a.num_heads * kBlockSize * kHeadDim;
  c.vdelta = (size_t)a.num_heads * kBlockSize * kHeadDim;
  c.k_head = a.pool + slab_offset(0, a.layer, 0, h / a.group, a.num_layers, a.num_heads);
  c.nb = (L + kBlockSize - 1) / kBlockSize;
  c.L = L;
  c.num_blocks = a.num_blocks;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int row = 4 * q + (lane >> 4);  // row of the block this lane's slot holds
    const int chunk = (lane & 15) ^ swz(row);  // the chunk the swizzle puts in slot lane & 15
    c.voff[q] = row * kRowBytes + chunk * 16;
  }

  // Stale LDS from earlier workgroups must never meet a zero weight as NaN.
  {
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < kTileBytes / 16; i += kPrefillThreads) {
      reinterpret_cast<uint4*>(g_k_tile0)[i] = z;
      reinterpret_cast<uint4*>(g_k_tile1)[i] = z;
      reinterpret_cast<uint4*>(g_k_tile2)[i] = z;
      reinterpret_cast<uint4*>(g_v_tile0)[i] = z;
      reinterpret_cast<uint4*>(g_v_tile1)[i] = z;
    }
  }

  // The wave's queries as MFMA B operands: Q[wq][16k + 8*half .. +7], k = 0..7.
  h8 qf[8];
  {
    const uint16_t* qrow = a.q + ((size_t)(qs0 + (q_ok ? wq : q_begin)) * a.num_q_heads + h) * kHeadDim + 8 * half;
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

  // Per-lane LDS offsets.  K operand (S^T = K Q^T): row 32T + col, chunk
  // 2k + half at position (2k + half) ^ swz(col).  V operand (O^T += V^T
  // P^T) through transposed reads: in each 16-lane group g, source lane s
  // points at key 16kk + 8r + 4(g >> 1) + s/4, dims 32dt + 16(g & 1) + 4(s & 3)
  // .. +3; the read hands lane i of the group the 4 keys of dim
  // 32dt + 16(g & 1) + i, matching the key order of P in S^T's registers.
  const int g = lane >> 4, sl = lane & 15;
  int v_row[2];
  int v_byte[2][4];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    v_row[rr] = 8 * rr + 4 * (g >> 1) + (sl >> 2);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = 32 * dt + 16 * (g & 1) + 4 * (sl & 3);
      v_byte[rr][dt] = v_row[rr] * kRowBytes + (((d >> 3) ^ swz(v_row[rr])) << 4) + (d & 7) * 2;
    }
  }

  // The work runs in half steps of 32 keys (rows 32T .. 32T+31 of a tile).
  // Scores of a half step in S^T's accumulator layout: register i of lane
  // (col, half) holds key 32T + 8(i/4) + 4*half + i%4 of query col.
  const float16_t zero = {};
  // S^T = K Q^T for one half step from a K tile.
  auto qk = [&](const char* kt, int T, float16_t& sc) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int pos = (2 * k + half) ^ swz(col);
      const h8 ka = *reinterpret_cast<const h8*>(kt + (32 * T + col) * kRowBytes + pos * 16);
      sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qf[k], k == 0 ? zero : sc, 0, 0, 0);
    }
  };
  // Keys after the query's position get -inf; kb is the half step's first key.
  auto mask = [&](float16_t& sc, int kb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = kb + 8 * (i >> 2) + 4 * half + (i & 3);
      if (key > p_q) sc[i] = -INFINITY;
    }
  };
  // The half step's largest scaled score of this lane's query (both lane halves).
  auto step_max = [&](const float16_t& sc) {
    float x = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) x = fmaxf(x, sc[i]);
    const auto both = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(both[0]), __uint_as_float(both[1])) * a.qk_scale;
  };
  // Weights 2^(s * scale - m) rounded to FP16 as the P*V operand, and their
  // row sum (of the FP16 values the product uses) accumulated in fp32.
  auto weights = [&](const float16_t& sc, h8* pb) {
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
    return ls;
  };
  // O^T += V^T P^T for one half step from a V tile: blocks 2T and 2T + 1.
  auto pv = [&](const h8* pb, const char* vt, int T) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const char* vb = vt + (2 * T + kk) * kBlockSize * kRowBytes;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS v4i16*)(vb + v_byte[0][dt]));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_LDS v4i16*)(vb + v_byte[1][dt]));
        const h8 va = bitcast<h8>(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pb[kk], o[dt], 0, 0, 0);
      }
    // Transposed V reads run two MFMAs ahead: four up front, then two (the
    // next MFMA's operand) after each MFMA while any remain.
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // one MFMA
      if (j < 6) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);  // two LDS reads
    }
  };
  // One half step: the QK^T of the next half step (into s_next) on the
  // matrix cores while this half step's softmax (of s_cur) runs on the
  // vector ALUs -- no branch in between, so the two interleave -- then this
  // half step's P*V.
  //
  // The exponent reference m moves only when a score exceeds it by more
  // than kLazy (log2 units).  Weights then stay below 2^kLazy, well inside
  // FP16, and the common half step computes its weights without waiting for
  // its own maximum.  O and the row sum are relative to the same m, so the
  // result is the same softmax; partial ranges carry m to the merge.
  constexpr float kLazy = 8.0f;
  auto half_step = [&](const char* kt_next, int t_next, float16_t& s_next, float16_t& s_cur, const char* vt, int t_cur) {
    qk(kt_next, t_next, s_next);
    const float mstep = step_max(s_cur);
    h8 pb[2];
    float ls = weights(s_cur, pb);
    // All eight K operand reads go out before the first MFMA that needs one:
    // the LDS latency then overlaps the chain instead of stalling each link.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // eight LDS reads
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
      __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);  // two transcendental
    }
    // Keep the common path's weights in this block: the rescale branch
    // overwrites them, and without this the compiler would move their
    // computation past the branch, away from the MFMAs it should overlap.
    asm volatile("" : "+v"(pb[0]), "+v"(pb[1]), "+v"(ls));
    if (__any(mstep > m + kLazy)) {
      const float mn = fmaxf(m, mstep);
      const float alpha = fast_exp2(m - mn);
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2) o[dt][r2] *= alpha;
      m = mn;
      ls = weights(s_cur, pb);
    }
    lsum += ls;
    pv(pb, vt, t_cur);
  };

  __syncthreads();  // zero fill done before any direct load lands
  const int nsteps = (k_end - k_begin + kBK - 1) / kBK;
  // Step i (64 keys): K in tile i % 3, V in tile i % 2.  Iteration i waits
  // for the loads issued one iteration earlier (K of step i+1, V of step i),
  // then refills the tiles nobody reads any more (K of step i+2 into the
  // tile of step i-1, V of step i+1 into the tile of step i-1), then runs
  // its two half steps; the second one's QK^T is the first half of step i+1.
  float16_t s0, s1;
  issue_rows(c, k_tile<0>(), k_begin, 0, false);
  issue_rows(c, v_tile<0>(), k_begin, 0, true);
  if (nsteps > 1) issue_rows(c, k_tile<1>(), k_begin + kBK, 1, false);
  loads_barrier();
  qk(k_tile<0>(), 0, s0);
  if (k_begin + 31 > p_wave_first) mask(s0, k_begin);
  auto iteration = [&](auto ktag, auto vtag, int i) {
    constexpr int SK = decltype(ktag)::value;  // i % 3
    constexpr int SV = decltype(vtag)::value;  // i % 2
    const int kb = k_begin + i * kBK;
    loads_barrier();
    if (i + 2 < nsteps) issue_rows(c, k_tile<(SK + 2) % 3>(), kb + 2 * kBK, i + 2, false);
    if (i + 1 < nsteps) issue_rows(c, v_tile<(SV + 1) % 2>(), kb + kBK, i + 1, true);
    half_step(k_tile<SK>(), 1, s1, s0, v_tile<SV>(), 0);
    if (kb + 63 > p_wave_first) mask(s1, kb + 32);
    // After the last step the next K tile holds an older step's keys (finite
    // values or zeros); those scores are never used.
    half_step(k_tile<(SK + 1) % 3>(), 0, s0, s1, v_tile<SV>(), 1);
    if (kb + 95 > p_wave_first) mask(s0, kb + 64);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  for (int i = 0; i < nsteps; i += 6) {
    iteration(I0(), I0(), i);
    if (i + 1 >= nsteps) break;
    iteration(I1(), I1(), i + 1);
    if (i + 2 >= nsteps) break;
    iteration(I2(), I0(), i + 2);
    if (i + 3 >= nsteps) break;
    iteration(I0(), I1(), i + 3);
    if (i + 4 >= nsteps) break;
    iteration(I1(), I0(), i + 4);
    if (i + 5 >= nsteps) break;
    iteration(I2(), I1(), i + 5);
  }

  {
    const auto both = __builtin_amdgcn_permlane32_swap(__float_as_uint(lsum), __float_as_uint(lsum), false, false);
    lsum = __uint_as_float(both[0]) + __uint_as_float(both[1]);
  }
  if (!q_ok) return;
  const int nsplit_q = p_q / kPrefillSplit + 1;
  if (kr == 0 && h == 0 && half == 0) a.tok_splits[qs0 + wq] = nsplit_q;
  if (kr >= nsplit_q) return;
  const size_t th = (size_t)(qs0 + wq) * a.num_q_heads + h;
  if (nsplit_q == 1) {
    const float inv = 1.0f / lsum;
    uint16_t* orow = a.out + th * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int d0 = 32 * dt + 8 * gq + 4 * half;
        uint2 w;
        w.x = pack_half2(o[dt][4 * gq] * inv, o[dt][4 * gq + 1] * inv);
        w.y = pack_half2(o[dt][4 * gq + 2] * inv, o[dt][4 * gq + 3] * inv);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
  } else {
    const size_t slot = th * a.max_splits + kr;
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
}

__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_mixed_kernel(PrefillArgs a) {
  // Workgroup n runs on XCD n % 8.  Along each XCD's sequence the prefill
  // tiles are spread evenly among the decode workgroups, so that a CU holds a
  // matrix-core-bound tile and a memory-bound decode group at the same time.
  // The prefill tiles an XCD gets are consecutive in (head, key range, query
  // tile) order, so the tiles that re-read one (head, key range) share its L2.
  const int n = blockIdx.x;
  const int x = n % kXcds;
  const int m = n / kXcds;
  const int np = a.prefill_wgs / kXcds;
  const int nd = a.decode_wgs / kXcds;
  const int tot = np + nd;
  int before, upto;
  if (a.interleave) {
    before = (int)((long long)m * np / tot);  // prefill positions before m
    upto = (int)((long long)(m + 1) * np / tot);
  } else {
    before = m < np ? m : np;  // all of an XCD's prefill tiles first
    upto = m < np ? m + 1 : np;
  }
  if (upto > before) {
    const int logical = x * np + before;
    const int tile = logical % a.tiles_max;
    const int rest = logical / a.tiles_max;
    const int kr = rest % a.ranges_max;
    const int h = rest / a.ranges_max;
    if (h >= a.num_q_heads) return;
    int row, qtile;
    if (!find_tile(a, tile, row, qtile)) return;
    prefill_tile(a, row, qtile, h, kr);
    return;
  }
  // decode rows: (row, 256-token range, group of kPrefillWaves query heads)
  // per workgroup.  Each wave folds its share of the range (as in the decode
  // launch) for every head of the group in turn, its loads running on from
  // one head to the next; after one barrier, wave w combines head w.  Each head's arithmetic is the decode launch's, so the
  // bits are too.  With grouping, the KV head is read once per query head.
  const int head_groups = (a.num_q_heads + kPrefillWaves - 1) / kPrefillWaves;
  const int d = (m - before) * kXcds + x;
  const int hg = d % head_groups;
  const int rs = d / head_groups;
  const int split = rs % a.max_splits;
  const int r = rs / a.max_splits;
  if (r >= a.num_rows) return;
  const int t = a.query_start[r];
  if (a.query_start[r + 1] - t != 1 || t < 0 || t >= a.total_q) return;
  int L = a.context_lens[r];
  L = L > a.max_context_len ? a.max_context_len : L;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h_own = hg * kPrefillWaves + wave;  // the head this wave combines
  if (split == 0 && hg == 0 && threadIdx.x == 0) a.tok_splits[t] = L < 1 ? 1 : decode_splits(L);
  if (L < 1) {
    if (split == 0 && h_own < a.num_q_heads && (threadIdx.x & 63) < 16)
      reinterpret_cast<uint4*>(a.out)[((size_t)t * a.num_q_heads + h_own) * 16 + (threadIdx.x & 15)] =
          make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int nsplit = decode_splits(L);
  if (split >= nsplit) return;
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int b0 = split * kSplitBlocks;
  const int b1 = min(nb, b0 + kSplitBlocks);
  // the shares are combined through the first K tile, which a decode workgroup does not use
  RangeScratch* lds = reinterpret_cast<RangeScratch*>(g_k_tile0);
  const int32_t* row_table = a.block_tables + (size_t)r * a.bt_stride;
  const int hq0 = hg * kPrefillWaves;
  const int nh = min(kPrefillWaves, a.num_q_heads - hq0);
  fold_share_heads<PKV_MIXED_DEPTH>(a.pool, a.layer, a.num_blocks, a.num_layers, a.num_heads, a.group, hq0, nh,
                                    row_table, L, b0, b1,
                                    reinterpret_cast<const uint4*>(a.q) + ((size_t)t * a.num_q_heads + hq0) * 16,
                                    a.qk_scale, lds);
  __syncthreads();
  if (h_own >= a.num_q_heads) return;
  const size_t th = (size_t)t * a.num_q_heads + h_own;
  const size_t slot = th * a.max_splits + split;
  combine_range(lds[wave], nsplit == 1, reinterpret_cast<uint32_t*>(a.out) + th * 64, a.part_o + slot * kHeadDim,
                a.part_ml + slot);
}

// One wave per (query token, head): merge the token's ranges when there is
// more than one.  The attention launch recorded each token's range count;
// a token it did not reach (a row that breaks the call's contract) reads a
// count clamped to the workspace, so its output is unspecified but every
// access stays inside the workspace.
__global__ __launch_bounds__(kPrefillThreads) void prefill_merge_kernel(PrefillArgs a) {
  const int t = blockIdx.x;
  const int h = __builtin_amdgcn_readfirstlane(blockIdx.y * kPrefillWaves + (threadIdx.x >> 6));
  if (h >= a.num_q_heads) return;
  int nsplit = a.tok_splits[t];
  nsplit = nsplit > a.max_splits ? a.max_splits : nsplit;
  if (nsplit <= 1) return;
  const size_t th = (size_t)t * a.num_q_heads + h;
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

extern "C" size_t pkv_prefill_workspace_size_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t num_rows,
                                                 int32_t total_q, int32_t max_q_per_row, int32_t max_context_len) {
  using namespace pkv;
  (void)num_rows;
  (void)max_q_per_row;
  if (!cache || total_q < 1 || max_context_len < 1 || cache->num_heads < 1 || num_q_heads < 1) return 0;
  const size_t n = (size_t)total_q * num_q_heads * prefill_max_splits(max_context_len);
  return align256(n * kHeadDim * sizeof(float)) + align256(n * sizeof(float2)) + align256((size_t)total_q * sizeof(int32_t));
}

extern "C" size_t pkv_prefill_workspace_size(const pkv_cache* cache, int32_t num_rows, int32_t total_q,
                                             int32_t max_q_per_row, int32_t max_context_len) {
  return cache ? pkv_prefill_workspace_size_gqa(cache, cache->num_heads, num_rows, total_q, max_q_per_row,
                                                max_context_len)
               : 0;
}

extern "C" int pkv_chunked_prefill_attention(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                             const int32_t* query_start, const int32_t* block_tables,
                                             int32_t bt_stride, const int32_t* context_lens, int32_t num_rows,
                                             int32_t total_q, int32_t max_q_per_row, int32_t max_context_len,
                                             float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!cache) return pkv::fail(PKV_ERR_INVALID_ARG, "cache is null");
  return pkv_chunked_prefill_attention_gqa(cache, cache->num_heads, layer, out, q, query_start, block_tables, bt_stride,
                                           context_lens, num_rows, total_q, max_q_per_row, max_context_len, scale,
                                           workspace, workspace_bytes, stream);
}

extern "C" int pkv_chunked_prefill_attention_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t layer, void* out,
                                                 const void* q, const int32_t* query_start,
                                                 const int32_t* block_tables, int32_t bt_stride,
                                                 const int32_t* context_lens, int32_t num_rows, int32_t total_q,
                                                 int32_t max_q_per_row, int32_t max_context_len, float scale,
                                                 void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (num_q_heads < 1 || num_q_heads % cache->num_heads || num_q_heads > 1024)
    return fail(PKV_ERR_UNSUPPORTED, "num_q_heads must be a multiple of the pool's KV heads (at most 1024)");
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
  const size_t need = pkv_prefill_workspace_size_gqa(cache, num_q_heads, num_rows, total_q, max_q_per_row, max_context_len);
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
  const size_t n = (size_t)total_q * num_q_heads * a.max_splits;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(workspace) + align256(n * kHeadDim * sizeof(float)));
  a.tok_splits = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + align256(n * kHeadDim * sizeof(float)) +
                                            align256(n * sizeof(float2)));
  a.layer = layer;
  a.num_blocks = cache->num_blocks;
  a.num_layers = cache->num_layers;
  a.num_heads = cache->num_heads;
  a.num_q_heads = num_q_heads;
  a.group = num_q_heads / cache->num_heads;
  a.bt_stride = bt_stride;
  a.num_rows = num_rows;
  a.total_q = total_q;
  a.max_context_len = max_context_len;
  a.qk_scale = scale * kLog2e;
  // Tiles: every row with n >= 2 wastes at most one partial tile, and rows
  // with n == 1 add none, so ceil(total_q / kBQ) + num_rows bounds the count.
  const int64_t tiles = max_q_per_row >= 2 ? ((int64_t)total_q + kBQ - 1) / kBQ + num_rows : 0;
  const int64_t ranges = ((int64_t)max_context_len + kPrefillSplit - 1) / kPrefillSplit;
  int64_t pre = tiles * ranges * num_q_heads;
  pre = (pre + kXcds - 1) / kXcds * kXcds;
  const int head_groups = (num_q_heads + kPrefillWaves - 1) / kPrefillWaves;
  int64_t dec = (int64_t)num_rows * decode_splits(max_context_len) * head_groups;
  dec = (dec + kXcds - 1) / kXcds * kXcds;
  if (pre + dec > INT32_MAX || tiles > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  a.tiles_max = (int)(tiles > 0 ? tiles : 1);
  a.ranges_max = (int)ranges;
  a.prefill_wgs = (int)pre;
  a.decode_wgs = (int)dec;
  // Spreading the tiles among the decode workgroups lets a CU hold a tile and
  // a decode workgroup at once, which pays when the batch has decode rows;
  // with none, the empty decode slots only scatter the tiles.  The host knows
  // no row's query count, but a batch whose rows are more than
  // ceil(total_q / max_q_per_row) cannot be all full-size chunks.  The choice
  // changes only the order of workgroups, never a result.
  const int64_t full_rows = ((int64_t)total_q + max_q_per_row - 1) / max_q_per_row;
  a.interleave = PKV_PREFILL_INTERLEAVE >= 0 ? PKV_PREFILL_INTERLEAVE : (num_rows > full_rows ? 1 : 0);
  hipStream_t s = static_cast<hipStream_t>(stream);
  prefill_mixed_kernel<<<dim3((unsigned)(pre + dec)), dim3(kPrefillThreads), 0, s>>>(a);
  if (int rc = check_launch("prefill mixed kernel")) return rc;
  prefill_merge_kernel<<<dim3((unsigned)total_q, (unsigned)head_groups), dim3(kPrefillThreads), 0, s>>>(a);
  return check_launch("prefill merge kernel");
}
