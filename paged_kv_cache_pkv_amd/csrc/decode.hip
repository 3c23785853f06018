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
// Mapping onto gfx950.  A workgroup of 4 waves owns one (row, head, range);
// wave w folds the range's w-th quarter (4 of its 16 blocks) and the waves
// combine their softmax states through LDS.  A 16-token block of one head is
// 4 KiB of keys followed (128 KiB later) by 4 KiB of values, stored
// [token][128].  Lane l works on dims 8*(l%16) .. +7 of tokens l/16, l/16 + 4,
// l/16 + 8, l/16 + 12: every load instruction moves four whole 256-byte token
// rows (1 KiB contiguous per wave), straight into registers -- each lane
// consumes exactly what it loads, so no LDS staging is needed.  Loads carry
// the non-temporal cache policy.  Scores are dot products of FP16 pairs
// accumulated in fp32 (v_dot2_f32_f16), summed over the 16 lanes of a token
// with DPP moves.  Each group of 16 lanes keeps its own online-softmax state
// over its four tokens of every block; the four groups merge at the end of the
// wave's share.  Blocks are software-pipelined two ahead.  Short shares keep
// many independent waves in flight, so the launch fills and drains faster
// than with one wave walking a whole range.

#include "decode_core.h"

namespace pkv {
namespace {

#ifndef PKV_XCD_REMAP
#define PKV_XCD_REMAP 1
#endif

constexpr int kWavesPerGroup = 4;  // heads per merge workgroup
constexpr int kDecodeThreads = 64 * kWavesPerGroup;
constexpr int kXcds = 8;
constexpr int kRowBytesGqm = kHeadDim * 2;  // one token row of one head

struct DecodeArgs {
  const uint16_t* pool;
  const uint4* q;       // [R][Hq][16] chunks of 8 halves
  uint4* out;           // [R][Hq][16]
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;        // [R][Hq][S][128]
  float2* part_ml;      // [R][Hq][S]
  const uint4* k_new;   // [R][H][16]: this step's new token per row (appending decode only)
  const uint4* v_new;
  int layer, num_blocks, num_layers, num_heads;  // num_heads: KV heads of the pool
  int num_q_heads;      // num_heads * G
  int bt_stride, num_rows, max_context_len, max_splits;
  float qk_scale;       // scale * log2(e)
};

// kAppend: each row's new token (position L - 1) comes from k_new / v_new and
// the range holding it also writes it into its pool slot (the step's append).
template <bool kAppend>
__global__ __launch_bounds__(64 * kRangeWaves) void decode_kernel(DecodeArgs a) {
  __shared__ RangeScratch lds;
  // 1-D grid over (row, range, head).  Workgroups go to the XCDs round-robin
  // by index; with the remap, the heads of one (row, range) land on one XCD
  // back to back, so they share its L2 and TLB for the same block slabs.
  const int n = blockIdx.x;
#if PKV_XCD_REMAP
  const int m = n / kXcds;
  const int h = m % a.num_heads;
  const int rs = (n % kXcds) + kXcds * (m / a.num_heads);
#else
  const int h = n % a.num_heads;
  const int rs = n / a.num_heads;
#endif
  const int split = rs % a.max_splits;
  const int r = rs / a.max_splits;
  if (r >= a.num_rows) return;
  const int L_in = a.context_lens[r];
  const int L = L_in > a.max_context_len ? a.max_context_len : L_in;
  const size_t rh = (size_t)r * a.num_heads + h;
  if (L < 1) {
    if (split == 0 && threadIdx.x < 16) a.out[rh * 16 + threadIdx.x] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int nsplit = decode_splits(L);
  if (split >= nsplit) return;
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int b0 = split * kSplitBlocks;
  const int b1 = min(nb, b0 + kSplitBlocks);
  const size_t slot = rh * a.max_splits + split;
  // A row longer than max_context_len is read clamped, for memory safety, but
  // its new token's slot lies past the clamp: it appends nothing.
  const bool app = kAppend && L_in == L;
  decode_range_waves(a.pool, a.layer, a.num_blocks, a.num_layers, a.num_heads, h,
                     a.block_tables + (size_t)r * a.bt_stride, L, b0, b1, nsplit == 1, a.q + rh * 16, a.qk_scale,
                     app ? a.k_new + rh * 16 : nullptr, app ? a.v_new + rh * 16 : nullptr,
                     reinterpret_cast<uint32_t*>(a.out) + rh * 64, a.part_o + slot * kHeadDim, a.part_ml + slot,
                     lds);
}

// Grouped-query decode: G query heads share each KV head.  A workgroup of
// kGqaWaves waves owns one (row, range, KV head); wave w folds its equal
// share of the range's 16 blocks for all G query heads, so every key and
// value is read once for the group, and the waves' softmax states combine
// through LDS in wave order (The inference engine, wpnews.pro: tile
// statistics combine exactly).  The range partition matches the decode
// launch's, so a row's result does not depend on its batch neighbours.
// Waves per workgroup by group size (each takes 16 / waves blocks of a range).
#ifndef PKV_GQA_WAVES2
#define PKV_GQA_WAVES2 2
#endif
#ifndef PKV_GQA_WAVES4
#define PKV_GQA_WAVES4 2
#endif
#ifndef PKV_GQA_WAVES8
#define PKV_GQA_WAVES8 2
#endif
#ifndef PKV_GQA_DEPTH
#define PKV_GQA_DEPTH 3
#endif
#ifndef PKV_GQA_DEPTH8
#define PKV_GQA_DEPTH8 2
#endif
template <int G>
constexpr int gqa_waves() {
  return G <= 2 ? PKV_GQA_WAVES2 : G <= 4 ? PKV_GQA_WAVES4 : PKV_GQA_WAVES8;
}

template <int G, bool kAppend>
__global__ __launch_bounds__(64 * gqa_waves<G>()) void decode_gqa_kernel(DecodeArgs a) {
  constexpr int kGqaWaves = gqa_waves<G>();
  static_assert(kSplitBlocks % kGqaWaves == 0, "each wave takes an equal share of a range");
  __shared__ float s_m[kGqaWaves][G], s_l[kGqaWaves][G];
  __shared__ float4 s_o[kGqaWaves][G][32];
  const int n = blockIdx.x;
#if PKV_XCD_REMAP
  // the KV heads of one (row, range) run back to back on one XCD
  const int m = n / kXcds;
  const int h = m % a.num_heads;
  const int rs = (n % kXcds) + kXcds * (m / a.num_heads);
#else
  const int h = n % a.num_heads;
  const int rs = n / a.num_heads;
#endif
  const int split = rs % a.max_splits;
  const int r = rs / a.max_splits;
  if (r >= a.num_rows) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int L_in = a.context_lens[r];
  const int L = L_in > a.max_context_len ? a.max_context_len : L_in;
  const size_t rh = (size_t)r * a.num_q_heads + (size_t)h * G;  // the KV head's first query head
  if (L < 1) {
    if (split == 0 && wave == 0 && lane < 16)
#pragma unroll
      for (int g = 0; g < G; ++g) a.out[(rh + g) * 16 + lane] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int nsplit = decode_splits(L);
  if (split >= nsplit) return;
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  constexpr int kPer = kSplitBlocks / kGqaWaves;
  const int b0 = min(nb, split * kSplitBlocks + wave * kPer);
  const int b1 = min(nb, b0 + kPer);
  SoftmaxState st[G];
  // with the append fused, the wave holding the row's last block takes the new token
  const uint4* new_k = nullptr;
  const uint4* new_v = nullptr;
  if constexpr (kAppend) {
    // a row clamped to max_context_len appends nothing (its slot lies past the clamp)
    if (b0 < b1 && b1 == nb && L_in == L) {
      new_k = a.k_new + ((size_t)r * a.num_heads + h) * 16;
      new_v = a.v_new + ((size_t)r * a.num_heads + h) * 16;
    }
  }
  fold_blocks<(G >= 8 ? PKV_GQA_DEPTH8 : PKV_GQA_DEPTH), G>(a.pool, a.layer, a.num_blocks, a.num_layers, a.num_heads, h,
                                        a.block_tables + (size_t)r * a.bt_stride, L, b0, b1, a.q + rh * 16,
                                        a.qk_scale, st, new_k, new_v);
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (lane < 16) {
      s_o[wave][g][2 * lane] = make_float4(st[g].o[0], st[g].o[1], st[g].o[2], st[g].o[3]);
      s_o[wave][g][2 * lane + 1] = make_float4(st[g].o[4], st[g].o[5], st[g].o[6], st[g].o[7]);
    }
    if (lane == 0) {
      s_m[wave][g] = st[g].m;
      s_l[wave][g] = st[g].l;
    }
  }
  __syncthreads();
  // wave w combines query heads g = w, w + kGqaWaves, ...; lane owns dims 2*lane, 2*lane + 1
  for (int g = wave; g < G; g += kGqaWaves) {
    float M = kMinusBig;
#pragma unroll
    for (int w = 0; w < kGqaWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float l = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kGqaWaves; ++w) {
      const float f = fast_exp2(s_m[w][g] - M);
      const float2 v = reinterpret_cast<const float2*>(&s_o[w][g][0])[lane];
      l = fmaf(s_l[w][g], f, l);
      o0 = fmaf(v.x, f, o0);
      o1 = fmaf(v.y, f, o1);
    }
    const size_t hq = rh + g;
    if (nsplit == 1) {
      const float inv = 1.0f / l;
      reinterpret_cast<uint32_t*>(a.out)[hq * 64 + lane] = pack_half2(o0 * inv, o1 * inv);
    } else {
      const size_t slot = hq * a.max_splits + split;
      reinterpret_cast<float2*>(a.part_o + slot * kHeadDim)[lane] = make_float2(o0, o1);
      if (lane == 0) a.part_ml[slot] = make_float2(M, l);
    }
  }
}

// Grouped-query decode on the matrix cores.  With G query heads per KV head
// the per-block work of a wave is two small matrix products, and on the
// vector ALUs it grows with G (the scores' lane reductions and P*V).  Here a
// 16-token block of one KV head folds into up to 16 query slots (G used, the
// rest zero) as:
//   S = K Q^T       v_mfma_f32_16x16x32_f16 x 4 (128 dims): A = the block's
//                   K rows, loaded from memory straight into the A layout
//                   (lane (g, t) holds dims 32c + 8g .. +7 of token t), B =
//                   the queries, held in registers for the whole range;
//   O^T += V^T P^T  v_mfma_f32_16x16x16_f16 x 8 (16 dims each): B = P^T,
//                   which is S's accumulator rounded to FP16 (lane (g, q)
//                   holds tokens 4g .. 4g+3 of query slot q), A = V^T, read
//                   from the block's V rows in LDS by ds_read_tr16_b64 (a
//                   16-lane group reads 4 rows x 16 dims and hands lane i the
//                   4 rows of dim i).
// V reaches LDS by direct global->LDS loads (no registers), K by ordinary
// loads into registers; each wave holds kGqmDepth blocks in its own LDS
// tiles and registers, one loading while one folds.  At two blocks the
// kernel fits 168 registers, three waves per SIMD; on the average mix with 8
// KV heads it takes 31 us per layer at G = 8 against 37 us for the vector
// fold, and ties it at G = 4 (45 us); at G = 2 the vector fold is faster
// (68 against 90 us), since 14 of the 16 query slots would be idle.  The
// online softmax is the grouped fold's: a lazy exponent reference
// (kGroupLazy) and FP16 weights whose rounded values also form the row sum.  Lane (g, q) keeps query slot q's statistics; the maximum over a
// block's 16 tokens is one exchange across the four lane groups.  Rows past
// the context read as zero through the buffer resource's range and get score
// -inf.  The range partition and the combine of the waves through LDS are
// the vector kernel's.
#ifndef PKV_GQM_WAVES
#define PKV_GQM_WAVES 4
#endif
#ifndef PKV_GQM_DEPTH
#define PKV_GQM_DEPTH 2
#endif
// group sizes from which the matrix-core kernel replaces the vector one
// (G = 4 and 8; G = 2 stays on the vector fold)
#ifndef PKV_GQA_MFMA_MIN_G
#define PKV_GQA_MFMA_MIN_G 4
#endif
constexpr int kGqmWaves = PKV_GQM_WAVES;
constexpr int kGqmDepth = PKV_GQM_DEPTH;
constexpr int kVTileBytes = kBlockSize * kHeadDim * 2;  // one block's V rows of one head
static_assert(kSplitBlocks % kGqmWaves == 0, "each wave takes an equal share of a range");
static_assert(kGqmDepth >= 2 && kGqmDepth <= 4, "blocks in flight per wave");

typedef short gqm_v4i16 __attribute__((ext_vector_type(4)));
#define PKV_GQM_LDS __attribute__((address_space(3)))

// Wait until at most N of this wave's vector memory operations are
// outstanding (they complete in issue order), and keep memory accesses from
// moving across the wait.
template <int N>
__device__ __forceinline__ void wait_vmem_at_most() {
  static_assert(N == 8 || N == 16 || N == 24, "eight operations per block");
  if constexpr (N == 8)
    asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else if constexpr (N == 16)
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else
    asm volatile("s_waitcnt vmcnt(24)" ::: "memory");
}

#ifndef PKV_GQM_OCC
#define PKV_GQM_OCC 1
#endif
template <int G, bool kAppend>
__global__ __launch_bounds__(64 * kGqmWaves, PKV_GQM_OCC) void decode_gqa_mfma_kernel(DecodeArgs a) {
  static_assert(G >= 2 && G <= 16, "the query slots of one 16-column product");
  constexpr int D = kGqmDepth;
  constexpr int kPer = kSplitBlocks / kGqmWaves;
  __shared__ __attribute__((aligned(16))) char s_tiles[kGqmWaves * D * kVTileBytes];
  __shared__ float s_m[kGqmWaves][G], s_l[kGqmWaves][G];
  static_assert(sizeof(float4) * kGqmWaves * G * 32 <= sizeof(s_tiles), "the combine reuses the V tiles");
  float4(*s_o)[G][32] = reinterpret_cast<float4(*)[G][32]>(s_tiles);
  const int n = blockIdx.x;
#if PKV_XCD_REMAP
  const int mx = n / kXcds;
  const int h = mx % a.num_heads;
  const int rs = (n % kXcds) + kXcds * (mx / a.num_heads);
#else
  const int h = n % a.num_heads;
  const int rs = n / a.num_heads;
#endif
  const int split = rs % a.max_splits;
  const int r = rs / a.max_splits;
  if (r >= a.num_rows) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int gg = lane >> 4;   // lane group: tokens 4gg .. 4gg+3 of S, dims 32c + 8gg of K
  const int col = lane & 15;  // token of K's A operand; query slot of S, P and O^T
  const int L_in = a.context_lens[r];
  const int L = L_in > a.max_context_len ? a.max_context_len : L_in;
  const size_t rh = (size_t)r * a.num_q_heads + (size_t)h * G;  // the KV head's first query head
  if (L < 1) {
    if (split == 0 && wave == 0 && lane < 16)
#pragma unroll
      for (int g = 0; g < G; ++g) a.out[(rh + g) * 16 + lane] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int nsplit = decode_splits(L);
  if (split >= nsplit) return;
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int b0 = min(nb, split * kSplitBlocks + wave * kPer);
  const int b1 = min(nb, b0 + kPer);

  // B operand of S = K Q^T: dims 32c + 8gg .. +7 of query slot col
  half8_t qb[4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
    qb[c] = col < G ? bitcast<half8_t>(a.q[(rh + col) * 16 + 4 * c + gg]) : half8_t{};

  const uint16_t* head_base = a.pool + slab_offset(0, a.layer, 0, h, a.num_layers, a.num_heads);
  const size_t block_stride = (size_t)a.num_layers * 2 * a.num_heads * kBlockSize * kHeadDim;
  const int vdelta = a.num_heads * kBlockSize * kHeadDim * 2;  // bytes from a head's K tile to its V tile
  const int32_t* row_table = a.block_tables + (size_t)r * a.bt_stride;
  const int my_id = (lane < b1 - b0) ? row_table[b0 + lane] : 0;
  // the V rows sit in LDS with chunk k of row t at chunk position k ^ (t & 15)
  int v_src[4];
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const int row = 4 * qd + gg;
    v_src[qd] = vdelta + row * kRowBytesGqm + ((col ^ (row & 15)) << 4);
  }
  const int tr_row = 4 * gg + (col >> 2);
  int tr_off[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const int dim = 16 * c + 4 * (col & 3);
    tr_off[c] = tr_row * kRowBytesGqm + (((dim >> 3) ^ (tr_row & 15)) << 4) + (dim & 7) * 2;
  }
  char* my_tiles = s_tiles + wave * D * kVTileBytes;

  // Issue block j's loads into slot `slot`: 4 K loads into registers, then 4
  // direct V loads into the slot's LDS tile.  Slots past the share issue the
  // same 8 operations on an empty range, so that every block is followed by
  // exactly D - 1 blocks' operations.
  half8_t kr[D][4];
  int rows_of[D];
  auto issue = [&](int slot, int j) {
    const bool live = j < b1;
    const int id = __builtin_amdgcn_readlane(my_id, live ? j - b0 : 0);
    const bool good = live && (unsigned)id < (unsigned)a.num_blocks;
    const int rows = good ? min(L - j * kBlockSize, kBlockSize) : 0;
    const uint16_t* base = head_base + (size_t)(good ? id : 0) * block_stride;
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(base), 0, good ? vdelta + rows * kRowBytesGqm : 0, 0x00020000);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      kr[slot][c] = bitcast<half8_t>(
          __builtin_amdgcn_raw_buffer_load_b128(rsrc, col * kRowBytesGqm + 64 * c + 16 * gg, 0, PKV_KV_CPOL));
#pragma unroll
    for (int qd = 0; qd < 4; ++qd)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (PKV_GQM_LDS void*)(my_tiles + slot * kVTileBytes + qd * 1024), 16,
                                               v_src[qd], 0, 0, PKV_KV_CPOL);
    rows_of[slot] = rows;
  };

  // with the append fused, the wave whose share ends at the row's last block takes the new token
  bool takes_new = false;
  if constexpr (kAppend) takes_new = b0 < b1 && b1 == nb && L_in == L;
  const int s_new = (L - 1) & (kBlockSize - 1);

  float4_t o[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) o[c] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m = kMinusBig, l = 0.0f;
  const half2_t ones = {(_Float16)1.0f, (_Float16)1.0f};

#pragma unroll
  for (int u = 0; u < D - 1; ++u) issue(u, b0 + u);
  for (int j = b0; j < b1; j += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int jj = j + u;
      if (jj < b1) {
        issue((u + D - 1) % D, jj + D - 1);
        wait_vmem_at_most<8 * (D - 1)>();  // block jj's K registers and V tile have landed
        char* tile = my_tiles + u * kVTileBytes;
        const int valid = rows_of[u];
        if (kAppend && takes_new && jj == nb - 1 && valid > 0) {
          const uint4* new_k = a.k_new + ((size_t)r * a.num_heads + h) * 16;
          const uint4* new_v = a.v_new + ((size_t)r * a.num_heads + h) * 16;
          if (col == s_new)
#pragma unroll
            for (int c = 0; c < 4; ++c) kr[u][c] = bitcast<half8_t>(new_k[4 * c + gg]);
          if (lane < 16) {
            const uint4 nk = new_k[lane], nv = new_v[lane];
            *reinterpret_cast<uint4*>(tile + s_new * kRowBytesGqm + ((lane ^ (s_new & 15)) << 4)) = nv;
            const int id = __builtin_amdgcn_readlane(my_id, jj - b0);
            uint16_t* slot_k = const_cast<uint16_t*>(head_base) + (size_t)id * block_stride + s_new * kHeadDim + lane * 8;
            *reinterpret_cast<uint4*>(slot_k) = nk;
            *reinterpret_cast<uint4*>(reinterpret_cast<char*>(slot_k) + vdelta) = nv;
          }
        }
        float4_t sc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int c = 0; c < 4; ++c) sc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kr[u][c], qb[c], sc, 0, 0, 0);
        if (valid < kBlockSize) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * gg + i >= valid) sc[i] = -INFINITY;
        }
        float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])) * a.qk_scale;
        mb = fmaxf(mb, shfl_xor(mb, 16));
        mb = fmaxf(mb, shfl_xor(mb, 32));
        if (__any(mb > m + kGroupLazy)) {
          const float mn = fmaxf(m, mb);
          const float alpha = fast_exp2(m - mn);
          l *= alpha;
#pragma unroll
          for (int c = 0; c < 8; ++c) o[c] *= alpha;
          m = mn;
        }
        half4_t pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[i] = (_Float16)fast_exp2(fmaf(sc[i], a.qk_scale, -m));
        l = __builtin_amdgcn_fdot2(half2_t{pb[2], pb[3]}, ones,
                                   __builtin_amdgcn_fdot2(half2_t{pb[0], pb[1]}, ones, l, false), false);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const gqm_v4i16 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16((PKV_GQM_LDS gqm_v4i16*)(tile + tr_off[c]));
          o[c] = __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<half4_t>(vt), pb, o[c], 0, 0, 0);
        }
      }
    }
  }
  l += shfl_xor(l, 16);
  l += shfl_xor(l, 32);
  // every direct load of this wave (the trailing empty ones too) has landed
  // and every LDS read has returned before the tiles become the combine's
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  __syncthreads();
  if (col < G) {
#pragma unroll
    for (int c = 0; c < 8; ++c) s_o[wave][col][4 * c + gg] = make_float4(o[c][0], o[c][1], o[c][2], o[c][3]);
    if (gg == 0) {
      s_m[wave][col] = m;
      s_l[wave][col] = l;
    }
  }
  __syncthreads();
  // wave w combines query heads g = w, w + kGqmWaves, ...; lane owns dims 2*lane, 2*lane + 1
  for (int g = wave; g < G; g += kGqmWaves) {
    float M = kMinusBig;
#pragma unroll
    for (int w = 0; w < kGqmWaves; ++w) M = fmaxf(M, s_m[w][g]);
    float lt = 0.0f, o0 = 0.0f, o1 = 0.0f;
#pragma unroll
    for (int w = 0; w < kGqmWaves; ++w) {
      const float f = fast_exp2(s_m[w][g] - M);
      const float2 v = reinterpret_cast<const float2*>(&s_o[w][g][0])[lane];
      lt = fmaf(s_l[w][g], f, lt);
      o0 = fmaf(v.x, f, o0);
      o1 = fmaf(v.y, f, o1);
    }
    const size_t hq = rh + g;
    if (nsplit == 1) {
      const float inv = 1.0f / lt;
      reinterpret_cast<uint32_t*>(a.out)[hq * 64 + lane] = pack_half2(o0 * inv, o1 * inv);
    } else {
      const size_t slot = hq * a.max_splits + split;
      reinterpret_cast<float2*>(a.part_o + slot * kHeadDim)[lane] = make_float2(o0, o1);
      if (lane == 0) a.part_ml[slot] = make_float2(M, lt);
    }
  }
}

// Merge the ranges of every (row, head) that has more than one; one wave per
// (row, head).
__global__ __launch_bounds__(kDecodeThreads) void decode_merge_kernel(DecodeArgs a) {
  const int r = blockIdx.x;
  const int h = __builtin_amdgcn_readfirstlane(blockIdx.y * kWavesPerGroup + (threadIdx.x >> 6));  // query head
  if (h >= a.num_q_heads) return;
  int L = a.context_lens[r];
  L = L > a.max_context_len ? a.max_context_len : L;
  if (L < 1) return;
  const int nsplit = decode_splits(L);
  if (nsplit <= 1) return;
  const size_t rh = (size_t)r * a.num_q_heads + h;
  merge_partials(a.part_o + rh * a.max_splits * kHeadDim, a.part_ml + rh * a.max_splits, nsplit,
                 reinterpret_cast<uint32_t*>(a.out) + rh * 64);
}

int max_splits_for(int32_t max_context_len) { return decode_splits(max_context_len); }

}  // namespace
}  // namespace pkv

extern "C" int32_t pkv_split_tokens(void) { return pkv::kSplitBlocks * pkv::kBlockSize; }

namespace pkv {
namespace {

int group_of(const pkv_cache* cache, int32_t num_q_heads) {
  if (num_q_heads < 1 || num_q_heads % cache->num_heads) return 0;
  const int g = num_q_heads / cache->num_heads;
  return (g == 1 || g == 2 || g == 4 || g == 8) ? g : 0;
}

}  // namespace
}  // namespace pkv

extern "C" size_t pkv_decode_workspace_size_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t num_rows,
                                                int32_t max_context_len) {
  using namespace pkv;
  if (!cache || num_rows < 1 || max_context_len < 1 || cache->num_heads < 1 || num_q_heads < 1) return 0;
  const size_t s = (size_t)max_splits_for(max_context_len);
  const size_t n = (size_t)num_rows * num_q_heads * s;
  return align256(n * kHeadDim * sizeof(float)) + align256(n * sizeof(float2));
}

extern "C" size_t pkv_decode_workspace_size(const pkv_cache* cache, int32_t num_rows, int32_t max_context_len) {
  return cache ? pkv_decode_workspace_size_gqa(cache, cache->num_heads, num_rows, max_context_len) : 0;
}

extern "C" int pkv_decode_attention(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                    const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                                    int32_t num_rows, int32_t max_context_len, float scale, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (!cache) return pkv::fail(PKV_ERR_INVALID_ARG, "cache is null");
  return pkv_decode_attention_gqa(cache, cache->num_heads, layer, out, q, block_tables, bt_stride, context_lens,
                                  num_rows, max_context_len, scale, workspace, workspace_bytes, stream);
}

namespace pkv {
namespace {

int decode_launch(const pkv_cache* cache, int32_t num_q_heads, int32_t layer, void* out, const void* q,
                  const void* k_new, const void* v_new, const int32_t* block_tables, int32_t bt_stride,
                  const int32_t* context_lens, int32_t num_rows, int32_t max_context_len, float scale,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (int rc = check_cache(cache)) return rc;
  const int G = group_of(cache, num_q_heads);
  if (!G) return fail(PKV_ERR_UNSUPPORTED, "num_q_heads must be 1, 2, 4 or 8 times the pool's KV heads");
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
  const size_t need = pkv_decode_workspace_size_gqa(cache, num_q_heads, num_rows, max_context_len);
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
  const size_t n = (size_t)num_rows * num_q_heads * ms;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = workspace ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + align256(n * kHeadDim * sizeof(float)))
                        : nullptr;
  a.k_new = static_cast<const uint4*>(k_new);
  a.v_new = static_cast<const uint4*>(v_new);
  a.layer = layer;
  a.num_blocks = cache->num_blocks;
  a.num_layers = cache->num_layers;
  a.num_heads = cache->num_heads;
  a.num_q_heads = num_q_heads;
  a.bt_stride = bt_stride;
  a.num_rows = num_rows;
  a.max_context_len = max_context_len;
  a.max_splits = ms;
  a.qk_scale = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int64_t rs_total = (int64_t)num_rows * ms;
#if PKV_XCD_REMAP
  rs_total = (rs_total + kXcds - 1) / kXcds * kXcds;
#endif
  if (G == 1) {
    const int64_t wgs = rs_total * cache->num_heads;
    if (wgs > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
    if (k_new)
      decode_kernel<true><<<dim3((unsigned)wgs), dim3(64 * kRangeWaves), 0, s>>>(a);
    else
      decode_kernel<false><<<dim3((unsigned)wgs), dim3(64 * kRangeWaves), 0, s>>>(a);
  } else {
    const int64_t wgs = rs_total * cache->num_heads;
    if (wgs > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
    const dim3 grid((unsigned)wgs);
    const dim3 mfma_block(64 * kGqmWaves);
    if (k_new) {
      if (G >= PKV_GQA_MFMA_MIN_G) {
        switch (G) {
          case 2: decode_gqa_mfma_kernel<2, true><<<grid, mfma_block, 0, s>>>(a); break;
          case 4: decode_gqa_mfma_kernel<4, true><<<grid, mfma_block, 0, s>>>(a); break;
          default: decode_gqa_mfma_kernel<8, true><<<grid, mfma_block, 0, s>>>(a); break;
        }
      } else {
        switch (G) {
          case 2: decode_gqa_kernel<2, true><<<grid, dim3(64 * gqa_waves<2>()), 0, s>>>(a); break;
          case 4: decode_gqa_kernel<4, true><<<grid, dim3(64 * gqa_waves<4>()), 0, s>>>(a); break;
          default: decode_gqa_kernel<8, true><<<grid, dim3(64 * gqa_waves<8>()), 0, s>>>(a); break;
        }
      }
    } else {
      if (G >= PKV_GQA_MFMA_MIN_G) {
        switch (G) {
          case 2: decode_gqa_mfma_kernel<2, false><<<grid, mfma_block, 0, s>>>(a); break;
          case 4: decode_gqa_mfma_kernel<4, false><<<grid, mfma_block, 0, s>>>(a); break;
          default: decode_gqa_mfma_kernel<8, false><<<grid, mfma_block, 0, s>>>(a); break;
        }
      } else {
        switch (G) {
          case 2: decode_gqa_kernel<2, false><<<grid, dim3(64 * gqa_waves<2>()), 0, s>>>(a); break;
          case 4: decode_gqa_kernel<4, false><<<grid, dim3(64 * gqa_waves<4>()), 0, s>>>(a); break;
          default: decode_gqa_kernel<8, false><<<grid, dim3(64 * gqa_waves<8>()), 0, s>>>(a); break;
        }
      }
    }
  }
  if (int rc = check_launch("decode split kernel")) return rc;
  if (ms > 1) {
    const int q_groups = (num_q_heads + kWavesPerGroup - 1) / kWavesPerGroup;
    decode_merge_kernel<<<dim3(num_rows, q_groups), dim3(kDecodeThreads), 0, s>>>(a);
    if (int rc = check_launch("decode merge kernel")) return rc;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_decode_attention_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t layer, void* out,
                                        const void* q, const int32_t* block_tables, int32_t bt_stride,
                                        const int32_t* context_lens, int32_t num_rows, int32_t max_context_len,
                                        float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return pkv::decode_launch(cache, num_q_heads, layer, out, q, nullptr, nullptr, block_tables, bt_stride, context_lens,
                            num_rows, max_context_len, scale, workspace, workspace_bytes, stream);
}

extern "C" int pkv_decode_attention_append_gqa(const pkv_cache* cache, int32_t num_q_heads, int32_t layer, void* out,
                                               const void* q, const void* k_new, const void* v_new,
                                               const int32_t* block_tables, int32_t bt_stride,
                                               const int32_t* context_lens, int32_t num_rows, int32_t max_context_len,
                                               float scale, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pkv;
  if (!cache) return fail(PKV_ERR_INVALID_ARG, "cache is null");
  if (!k_new || !v_new) return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  return decode_launch(cache, num_q_heads, layer, out, q, k_new, v_new, block_tables, bt_stride, context_lens,
                       num_rows, max_context_len, scale, workspace, workspace_bytes, stream);
}

extern "C" int pkv_decode_attention_append(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                           const void* k_new, const void* v_new, const int32_t* block_tables,
                                           int32_t bt_stride, const int32_t* context_lens, int32_t num_rows,
                                           int32_t max_context_len, float scale, void* workspace,
                                           size_t workspace_bytes, void* stream) {
  if (!cache) return pkv::fail(PKV_ERR_INVALID_ARG, "cache is null");
  return pkv_decode_attention_append_gqa(cache, cache->num_heads, layer, out, q, k_new, v_new, block_tables, bt_stride,
                                         context_lens, num_rows, max_context_len, scale, workspace, workspace_bytes,
                                         stream);
}

// ---------------------------------------------------------------- no-alloc call
//
// pkv_decode_attention_append for callers that cannot allocate (code under HIP
// graph capture, tight serving loops): the split-K partials live in this
// library-owned device array instead of a caller workspace.  Each GPU holds
// its own copy of the array until the process ends; its device address is
// looked up once per device (the array's name is a host-side stand-in and
// must never reach a kernel).  Calls on one GPU share the array: calls that
// overlap in time on one GPU race.  Nothing in it needs clearing: a call
// writes every partial it reads.

#include <atomic>
#include <mutex>

namespace pkv {
namespace {

constexpr size_t kScratchBytes = PKV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mutex;

// The current device's copy of `scratch` (its device address), or null with
// the error set.
void* scratch_on_current_device() {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(PKV_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(PKV_ERR_UNSUPPORTED, "device index beyond the library's scratch table");
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || !p) {
      fail(PKV_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(g));
      return nullptr;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_decode_attention_append_noalloc(const pkv_cache* cache, int32_t layer, void* out, const void* q,
                                                   const void* k_new, const void* v_new,
                                                   const int32_t* block_tables, int32_t bt_stride,
                                                   const int32_t* context_lens, int32_t num_rows,
                                                   int32_t max_context_len, float scale, void* stream) {
  using namespace pkv;
  if (int rc = check_cache(cache)) return rc;
  if (num_rows < 1 || max_context_len < 1) return fail(PKV_ERR_INVALID_ARG, "num_rows and max_context_len must be >= 1");
  const size_t need = pkv_decode_workspace_size(cache, num_rows, max_context_len);
  if (need > kScratchBytes)
    return fail(PKV_ERR_WORKSPACE, "the call needs " + std::to_string(need) +
                                       " bytes of split-K scratch; the no-alloc call holds at most " +
                                       std::to_string(kScratchBytes) + " (use pkv_decode_attention_append)");
  void* ws = scratch_on_current_device();
  if (!ws) return PKV_ERR_HIP;
  return pkv_decode_attention_append(cache, layer, out, q, k_new, v_new, block_tables, bt_stride, context_lens,
                                     num_rows, max_context_len, scale, ws, kScratchBytes, stream);
}
