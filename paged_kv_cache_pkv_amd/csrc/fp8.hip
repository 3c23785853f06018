// 8-bit KV cache: append that quantizes, decode that reads codes.
//
// An 8-bit cache halves the bytes of every cached token and the attention
// read traffic, at a quality cost that grows with context length (Inference
// Infrastructure, seeitflow.com, its paragraph on KV-cache precision; The inference engine,
// wpnews.pro, "IO-aware attention and quantization attack different costs").
// Codes are FP8 E4M3 (the OCP format gfx950 converts natively), with one fp32
// scale per (token, head) row of 128 values: s = amax / 448 and codes encode
// x * (448 / amax), rounded to the nearest code with ties to the even
// mantissa and saturated at 448.  The scale is fixed when the token is
// appended, so earlier tokens of a block never need requantizing.
//
// Pool: codes [block][layer][2][head][16][128] bytes (the FP16 layout at one
// byte per value) and scales [block][layer][2][head][16] fp32.  Per token and
// layer 2 x heads x (128 + 4) bytes are read: 8,448 B at 32 heads instead of
// 16,384.
//
// Decode keeps the FP16 kernel's work split (one workgroup of four waves per
// (row, head, range), the waves' states combined through LDS, XCD-aware
// order, the same merge), over 512-token ranges, with one change of lane
// layout: lane group g holds tokens 4g .. 4g+3 of each block, so its four
// scales are one 16-byte load.  K codes widen to fp32
// exactly (v_cvt_pk_f32_fp8); the K scale multiplies the score and the V
// scale the softmax weight.

#include "decode_core.h"

namespace pkv {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Two 8-bit blocks in registers per wave (one loading while one folds) keep
// a wave at 112-118 registers, so four waves fit each SIMD: a CU then holds
// four 4-wave workgroups, 16 waves with 32 blocks in flight.  Three blocks
// per wave (three waves per SIMD) measured 2-4% slower on the average mix.
#ifndef PKV_F8_DEPTH
#define PKV_F8_DEPTH 2
#endif

constexpr int kRowCodes = kHeadDim;  // bytes of one (token, head) row
#ifndef PKV_F8_SPLIT_BLOCKS
#define PKV_F8_SPLIT_BLOCKS 32
#endif
// Blocks per split-K range: 512 tokens.  An 8-bit block moves half the bytes
// of an FP16 one, so a range holds twice the FP16 range's blocks for about the
// same bytes; each of the range's four waves folds 8 of them.  On the average
// mix 32 blocks measured 67-71 us per layer against 73-80 at 16 blocks and
// 77-79 at 64.
constexpr int kF8SplitBlocks = PKV_F8_SPLIT_BLOCKS;
static_assert(kF8SplitBlocks >= 1 && kF8SplitBlocks <= 64, "a range's block ids must fit one wave");
#ifndef PKV_F8_RANGE_WAVES
#define PKV_F8_RANGE_WAVES 4
#endif
constexpr int kF8RangeWaves = PKV_F8_RANGE_WAVES;  // waves that share one range
static_assert(kF8SplitBlocks % kF8RangeWaves == 0, "each wave takes an equal share of a range");
__host__ __device__ constexpr int f8_splits(int L) {
  return ((L + kBlockSize - 1) / kBlockSize + kF8SplitBlocks - 1) / kF8SplitBlocks;
}
constexpr int kF8DecodeThreads = 64 * kF8RangeWaves;  // one range's waves
constexpr int kF8MergeWaves = 4;                     // heads per merge workgroup, one wave each
constexpr int kF8MergeThreads = 64 * kF8MergeWaves;
constexpr int kF8Xcds = 8;

struct Cache8 {
  uint8_t* codes;
  float* scales;
  int num_blocks, num_layers, num_heads;
};

// Offset (in rows of 128 codes, or in scales) of (block, layer, kv, head, slot).
__device__ __host__ __forceinline__ size_t row_index(int b, int l, int kv, int h, int s, int num_layers, int num_heads) {
  return ((((size_t)b * num_layers + l) * 2 + kv) * num_heads + h) * kBlockSize + s;
}

// Nearest E4M3 code of x (ties to the even mantissa), magnitudes >= 448
// saturated.  All steps are exact fp32 operations plus two round-to-nearest-
// even roundings, so the result is reproducible bit for bit.
__device__ __forceinline__ uint32_t encode_e4m3(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 31) << 7;
  const float a = fabsf(x);
  if (a >= 448.0f) return sign | 0x7Eu;
  if (a < 0x1p-6f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);  // multiples of 2^-9; 8 is code 0x08
  int ex;
  (void)__builtin_frexpf(a, &ex);  // a = mant * 2^ex, mant in [0.5, 1)
  int e = ex - 1;
  int m = (int)__builtin_rintf((__builtin_ldexpf(a, -e) - 1.0f) * 8.0f);
  if (m == 8) {
    m = 0;
    e += 1;
  }
  return sign | (uint32_t)((e + 7) << 3) | (uint32_t)m;
}

// One workgroup per new token; 16 lanes per (kv, head) row, 8 values each.
constexpr int kAppendThreads = 256;

// Maximum over each aligned group of 16 lanes (one DPP row); every lane of
// the group receives it.
__device__ __forceinline__ float max16(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));   // lane ^ 1
  v = fmaxf(v, dpp_mov<0x4E>(v));   // lane ^ 2
  v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
  return v;
}

// Quantize one (token, head) row held by a 16-lane group (8 values per lane):
// the row's amax over the group, the lane's 8 codes, and the row's scale.
__device__ __forceinline__ u32x2 quantize_row8(const uint4& raw, float& scale) {
  float x[8];
  unpack8(raw, x);
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = max16(amax);
  const float inv = amax > 0.0f ? 448.0f / amax : 0.0f;
  uint32_t lo = 0, hi = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) lo |= (amax > 0.0f ? encode_e4m3(x[e] * inv) : 0u) << (8 * e);
#pragma unroll
  for (int e = 0; e < 4; ++e) hi |= (amax > 0.0f ? encode_e4m3(x[4 + e] * inv) : 0u) << (8 * e);
  scale = amax > 0.0f ? amax / 448.0f : 0.0f;
  return u32x2{lo, hi};
}

// One workgroup per (new token, 16 of its 2 * num_heads K/V rows): 16 lanes
// per row take 8 values each.  Every (token, row) is independent, so all of a
// step's rows run at once rather than in passes behind each other's loads.
__global__ __launch_bounds__(kAppendThreads) void append_fp8_kernel(
    Cache8 c, int layer, const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
    const int32_t* __restrict__ positions, const int32_t* __restrict__ request_of_token,
    const int32_t* __restrict__ block_tables, int num_rows, int bt_stride) {
  const int t = blockIdx.x;
  const int row = blockIdx.y * (kAppendThreads / 16) + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  const int rows = 2 * c.num_heads;
  if (row >= rows) return;  // whole 16-lane groups leave together
  const int kv = row / c.num_heads;
  const int h = row % c.num_heads;
  // the token's values first: their load overlaps the dependent reads of the
  // row, the position and the block id
  const uint4 raw = (kv ? v_new : k_new)[((size_t)t * c.num_heads + h) * 16 + part];
  const int r = request_of_token[t];
  const int p = positions[t];
  if (r < 0 || r >= num_rows || p < 0 || (p >> 4) >= bt_stride) return;
  const int b = block_tables[(size_t)r * bt_stride + (p >> 4)];
  if (b < 0 || b >= c.num_blocks) return;
  const int slot = p & 15;
  float scale;
  const u32x2 codes = quantize_row8(raw, scale);
  const size_t ri = row_index(b, layer, kv, h, slot, c.num_layers, c.num_heads);
  *reinterpret_cast<u32x2*>(c.codes + ri * kRowCodes + part * 8) = codes;
  if (part == 0) c.scales[ri] = scale;
}

struct F8Tile {
  u32x2 k[4];   // codes of tokens 4g+i, dims 8*chunk .. +7
  u32x2 v[4];
  float4 sk;    // scales of tokens 4g .. 4g+3
  float4 sv;
};

struct F8Args {
  Cache8 c;
  const uint4* q;   // [R][H][16]
  uint4* out;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_o;
  float2* part_ml;
  const uint4* k_new;  // [R][H][16] FP16: each row's new token (appending decode only)
  const uint4* v_new;
  int layer, bt_stride, num_rows, max_context_len, max_splits;
  float qk_scale;
};

__device__ __forceinline__ void load_f8_tile(F8Tile& t, const Cache8& c, int b, int layer, int h, int group, int chunk) {
  const size_t rk = row_index(b, layer, 0, h, 4 * group, c.num_layers, c.num_heads);
  const size_t rv = row_index(b, layer, 1, h, 4 * group, c.num_layers, c.num_heads);
  const uint8_t* kc = c.codes + rk * kRowCodes + chunk * 8;
  const uint8_t* vc = c.codes + rv * kRowCodes + chunk * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    t.k[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(kc + i * kRowCodes));
    t.v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(vc + i * kRowCodes));
  }
  t.sk = *reinterpret_cast<const float4*>(c.scales + rk);
  t.sv = *reinterpret_cast<const float4*>(c.scales + rv);
}

__device__ __forceinline__ void codes8_to_f32(u32x2 w, float* out) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[0], false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[0], true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[1], false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[1], true);
  out[0] = a[0]; out[1] = a[1]; out[2] = b[0]; out[3] = b[1];
  out[4] = c[0]; out[5] = c[1]; out[6] = d[0]; out[7] = d[1];
}

// Dot product of eight FP16 query values with eight E4M3 codes.  Every E4M3
// value is exact in FP16, so the codes are widened to packed halves (scale
// exponent 0) and multiplied with the two-term FP16 dot, accumulating in fp32.
__device__ __forceinline__ float dot8_f8(const uint4& q, u32x2 w) {
  float acc = 0.0f;
  acc = __builtin_amdgcn_fdot2(bitcast<half2_t>(q.x), __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, false), acc,
                               false);
  acc = __builtin_amdgcn_fdot2(bitcast<half2_t>(q.y), __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[0], 1.0f, true), acc,
                               false);
  acc = __builtin_amdgcn_fdot2(bitcast<half2_t>(q.z), __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, false), acc,
                               false);
  acc = __builtin_amdgcn_fdot2(bitcast<half2_t>(q.w), __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w[1], 1.0f, true), acc,
                               false);
  return acc;
}

// Fold one block (16 tokens; this lane's group holds tokens 4*group .. +3)
// into the group's running softmax state.  Tail is set only for a block with
// fewer than 16 live tokens (the row's last block, or an invalid id): its dead
// tokens get score -inf and weight 0, and their codes are cleared, because
// stale slots may hold NaN codes and scales (0 * NaN would leak).
template <bool Tail>
__device__ __forceinline__ void fold_f8(SoftmaxState& st, F8Tile& t, const uint4& q, float qk_scale, int group,
                                        int valid) {
  const float skv[4] = {t.sk.x, t.sk.y, t.sk.z, t.sk.w};
  const float svv[4] = {t.sv.x, t.sv.y, t.sv.z, t.sv.w};
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = sum16(dot8_f8(q, t.k[i])) * skv[i] * qk_scale;
  bool live[4] = {true, true, true, true};
  if (Tail) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      live[i] = 4 * group + i < valid;
      if (!live[i]) {
        s[i] = -INFINITY;
        t.v[i] = u32x2{0u, 0u};
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
  float pw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pw[i] = (!Tail || live[i]) ? p[i] * svv[i] : 0.0f;
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) codes8_to_f32(t.v[i], v[i]);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc = st.o[e] * alpha;
    acc = fmaf(pw[0], v[0][e], acc);
    acc = fmaf(pw[1], v[1][e], acc);
    acc = fmaf(pw[2], v[2][e], acc);
    acc = fmaf(pw[3], v[3][e], acc);
    st.o[e] = acc;
  }
  st.m = mn;
}

// kAppend: the wave whose share of a range ends at the row's last block
// quantizes the row's new token from k_new / v_new exactly as pkv_append_fp8
// does, folds those codes and scales in place of the slot's stale ones, and
// writes them into the slot.
template <bool kAppend>
__global__ __launch_bounds__(kF8DecodeThreads) void decode_fp8_kernel(F8Args a) {
  // one workgroup per (row, range, head); heads of a (row, range) back to back on one XCD
  __shared__ RangeScratchW<kF8RangeWaves> lds;
  const int n = blockIdx.x;
  const int mq = n / kF8Xcds;
  const int h = mq % a.c.num_heads;
  const int rs = (n % kF8Xcds) + kF8Xcds * (mq / a.c.num_heads);
  const int split = rs % a.max_splits;
  const int r = rs / a.max_splits;
  if (r >= a.num_rows) return;
  const int L_in = a.context_lens[r];
  const int L = L_in > a.max_context_len ? a.max_context_len : L_in;
  const int lane = threadIdx.x & 63;
  const int group = lane >> 4;
  const int chunk = lane & 15;
  const size_t rh = (size_t)r * a.c.num_heads + h;
  if (L < 1) {
    if (split == 0 && threadIdx.x < 16) a.out[rh * 16 + lane] = make_uint4(0u, 0u, 0u, 0u);
    return;
  }
  const int nb = (L + kBlockSize - 1) / kBlockSize;
  const int nsplit = f8_splits(L);
  if (split >= nsplit) return;
  // wave w folds the w-th equal share of the range; the states combine below
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int kPer = kF8SplitBlocks / kF8RangeWaves;
  const int rb0 = split * kF8SplitBlocks;
  const int rb1 = min(nb, rb0 + kF8SplitBlocks);
  const int b0 = min(rb1, rb0 + wave * kPer);
  const int b1 = min(rb1, b0 + kPer);
  const int32_t* row_table = a.block_tables + (size_t)r * a.bt_stride;
  const int my_id = (lane < b1 - b0) ? row_table[b0 + lane] : 0;
  const uint4 q = a.q[rh * 16 + chunk];
  SoftmaxState st;
  st.m = kMinusBig;
  st.l = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) st.o[e] = 0.0f;

  // the new token (slot ns of the last block: group ns / 4, entry ns % 4),
  // taken by the wave whose blocks end at the row's last block; a row clamped
  // to max_context_len appends nothing (its slot lies past the clamp)
  const bool takes_new = kAppend && b0 < b1 && b1 == nb && L_in == L;
  const int ns = (L - 1) & (kBlockSize - 1);
  u32x2 nkc = u32x2{0u, 0u}, nvc = nkc;
  float nks = 0.0f, nvs = 0.0f;
  if (takes_new) {
    nkc = quantize_row8(a.k_new[rh * 16 + chunk], nks);
    nvc = quantize_row8(a.v_new[rh * 16 + chunk], nvs);
  }
  constexpr int D = PKV_F8_DEPTH;  // blocks in registers: D - 1 loading while one folds
  F8Tile tile[D];
  bool ok[D];
  auto issue = [&](F8Tile& t, bool& good, int j) {
    const int id = __builtin_amdgcn_readlane(my_id, j - b0);
    good = (unsigned)id < (unsigned)a.c.num_blocks;
    load_f8_tile(t, a.c, good ? id : 0, a.layer, h, group, chunk);
  };
#pragma unroll
  for (int u = 0; u < D - 1; ++u)
    if (b0 + u < b1) issue(tile[u], ok[u], b0 + u);
  for (int j = b0; j < b1; j += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int jj = j + u;
      if (jj + D - 1 < b1) issue(tile[(u + D - 1) % D], ok[(u + D - 1) % D], jj + D - 1);
      if (jj < b1) {
        const int valid = ok[u] ? min(L - jj * kBlockSize, kBlockSize) : 0;
        if (takes_new && jj == nb - 1 && ok[u] && group == (ns >> 2)) {
          const int e = ns & 3;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i == e) {
              tile[u].k[i] = nkc;
              tile[u].v[i] = nvc;
            }
          tile[u].sk.x = e == 0 ? nks : tile[u].sk.x;
          tile[u].sk.y = e == 1 ? nks : tile[u].sk.y;
          tile[u].sk.z = e == 2 ? nks : tile[u].sk.z;
          tile[u].sk.w = e == 3 ? nks : tile[u].sk.w;
          tile[u].sv.x = e == 0 ? nvs : tile[u].sv.x;
          tile[u].sv.y = e == 1 ? nvs : tile[u].sv.y;
          tile[u].sv.z = e == 2 ? nvs : tile[u].sv.z;
          tile[u].sv.w = e == 3 ? nvs : tile[u].sv.w;
          const int id = __builtin_amdgcn_readlane(my_id, jj - b0);
          const size_t rk = row_index(id, a.layer, 0, h, ns, a.c.num_layers, a.c.num_heads);
          const size_t rv = row_index(id, a.layer, 1, h, ns, a.c.num_layers, a.c.num_heads);
          *reinterpret_cast<u32x2*>(a.c.codes + rk * kRowCodes + chunk * 8) = nkc;
          *reinterpret_cast<u32x2*>(a.c.codes + rv * kRowCodes + chunk * 8) = nvc;
          if (chunk == 0) {
            a.c.scales[rk] = nks;
            a.c.scales[rv] = nvs;
          }
        }
        if (valid == kBlockSize)
          fold_f8<false>(st, tile[u], q, a.qk_scale, group, valid);
        else
          fold_f8<true>(st, tile[u], q, a.qk_scale, group, valid);
      }
    }
  }
  merge_groups(st);
  store_share(st, lds, wave);
  __syncthreads();
  if (wave == 0) {
    const size_t slot = rh * a.max_splits + split;
    combine_range(lds, nsplit == 1, reinterpret_cast<uint32_t*>(a.out) + rh * 64, a.part_o + slot * kHeadDim,
                  a.part_ml + slot);
  }
}

__global__ __launch_bounds__(kF8MergeThreads) void merge_fp8_kernel(F8Args a) {
  const int r = blockIdx.x;
  const int h = __builtin_amdgcn_readfirstlane(blockIdx.y * kF8MergeWaves + (threadIdx.x >> 6));
  if (h >= a.c.num_heads) return;
  int L = a.context_lens[r];
  L = L > a.max_context_len ? a.max_context_len : L;
  if (L < 1) return;
  const int nsplit = f8_splits(L);
  if (nsplit <= 1) return;
  const size_t rh = (size_t)r * a.c.num_heads + h;
  merge_partials(a.part_o + rh * a.max_splits * kHeadDim, a.part_ml + rh * a.max_splits, nsplit,
                 reinterpret_cast<uint32_t*>(a.out) + rh * 64);
}

int check_cache8(const pkv_cache8* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARG, "cache is null");
  if (!c->codes || !c->scales) return fail(PKV_ERR_INVALID_ARG, "cache->codes and cache->scales must be set");
  if (c->block_size != kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "only block_size 16 is supported");
  if (c->head_dim != kHeadDim) return fail(PKV_ERR_UNSUPPORTED, "only head_dim 128 is supported");
  if (c->num_heads < 1 || c->num_heads > 128) return fail(PKV_ERR_UNSUPPORTED, "num_heads must be in [1, 128]");
  if (c->num_blocks < 1 || c->num_layers < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks and num_layers must be >= 1");
  if ((reinterpret_cast<uintptr_t>(c->codes) | reinterpret_cast<uintptr_t>(c->scales)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "cache->codes and cache->scales must be 16-byte aligned");
  return PKV_OK;
}

Cache8 cache8_of(const pkv_cache8* c) {
  Cache8 k;
  k.codes = static_cast<uint8_t*>(c->codes);
  k.scales = static_cast<float*>(c->scales);
  k.num_blocks = c->num_blocks;
  k.num_layers = c->num_layers;
  k.num_heads = c->num_heads;
  return k;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_append_fp8(const pkv_cache8* cache, int32_t layer, const void* k_new, const void* v_new,
                              const int32_t* positions, const int32_t* request_of_token, int32_t num_tokens,
                              const int32_t* block_tables, int32_t num_rows, int32_t bt_stride, void* stream) {
  using namespace pkv;
  if (int rc = check_cache8(cache)) return rc;
  if (layer < 0 || layer >= cache->num_layers) return fail(PKV_ERR_INVALID_ARG, "layer out of range");
  if (num_tokens < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_tokens == 0) {
    clear_error();
    return PKV_OK;
  }
  if (!k_new || !v_new || !positions || !request_of_token || !block_tables)
    return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (num_rows < 1 || bt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "num_rows and bt_stride must be >= 1");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  const unsigned row_groups = (unsigned)((2 * cache->num_heads + kAppendThreads / 16 - 1) / (kAppendThreads / 16));
  append_fp8_kernel<<<dim3(num_tokens, row_groups), dim3(kAppendThreads), 0, static_cast<hipStream_t>(stream)>>>(
      cache8_of(cache), layer, static_cast<const uint4*>(k_new), static_cast<const uint4*>(v_new), positions,
      request_of_token, block_tables, num_rows, bt_stride);
  return check_launch("pkv_append_fp8");
}

extern "C" size_t pkv_decode_workspace_size_fp8(const pkv_cache8* cache, int32_t num_rows, int32_t max_context_len) {
  using namespace pkv;
  if (!cache || num_rows < 1 || max_context_len < 1 || cache->num_heads < 1) return 0;
  const size_t s = (size_t)f8_splits(max_context_len);
  const size_t n = (size_t)num_rows * cache->num_heads * s;
  return align256(n * kHeadDim * sizeof(float)) + align256(n * sizeof(float2));
}

namespace pkv {
namespace {

int decode_fp8_launch(const pkv_cache8* cache, int32_t layer, void* out, const void* q, const void* k_new,
                      const void* v_new, const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                      int32_t num_rows, int32_t max_context_len, float scale, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (int rc = check_cache8(cache)) return rc;
  if (layer < 0 || layer >= cache->num_layers) return fail(PKV_ERR_INVALID_ARG, "layer out of range");
  if (num_rows < 1) return fail(PKV_ERR_INVALID_ARG, "num_rows must be >= 1");
  if (!out || !q || !block_tables || !context_lens) return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if (bt_stride < 1) return fail(PKV_ERR_INVALID_ARG, "bt_stride must be >= 1");
  if (max_context_len < 1 || (int64_t)max_context_len > (int64_t)bt_stride * kBlockSize)
    return fail(PKV_ERR_INVALID_ARG, "max_context_len must be in [1, bt_stride * 16]");
  if (!(scale > 0.0f) || !__builtin_isfinite(scale)) return fail(PKV_ERR_INVALID_ARG, "scale must be finite and > 0");
  if ((reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(q)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "out and q must be 16-byte aligned");
  const int ms = f8_splits(max_context_len);
  const size_t need = pkv_decode_workspace_size_fp8(cache, num_rows, max_context_len);
  if (ms > 1) {
    if (!workspace || workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
    if (reinterpret_cast<uintptr_t>(workspace) & 255) return fail(PKV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  F8Args a;
  a.c = cache8_of(cache);
  a.q = static_cast<const uint4*>(q);
  a.out = static_cast<uint4*>(out);
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t n = (size_t)num_rows * cache->num_heads * ms;
  a.part_o = static_cast<float*>(workspace);
  a.part_ml = workspace ? reinterpret_cast<float2*>(static_cast<char*>(workspace) + align256(n * kHeadDim * sizeof(float)))
                        : nullptr;
  a.k_new = static_cast<const uint4*>(k_new);
  a.v_new = static_cast<const uint4*>(v_new);
  a.layer = layer;
  a.bt_stride = bt_stride;
  a.num_rows = num_rows;
  a.max_context_len = max_context_len;
  a.max_splits = ms;
  a.qk_scale = scale * kLog2e;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int head_groups = (cache->num_heads + kF8MergeWaves - 1) / kF8MergeWaves;
  int64_t rs_total = ((int64_t)num_rows * ms + kF8Xcds - 1) / kF8Xcds * kF8Xcds;
  const int64_t wgs = rs_total * cache->num_heads;
  if (wgs > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "grid too large");
  if (k_new)
    decode_fp8_kernel<true><<<dim3((unsigned)wgs), dim3(kF8DecodeThreads), 0, s>>>(a);
  else
    decode_fp8_kernel<false><<<dim3((unsigned)wgs), dim3(kF8DecodeThreads), 0, s>>>(a);
  if (int rc = check_launch("decode fp8 kernel")) return rc;
  if (ms > 1) {
    merge_fp8_kernel<<<dim3(num_rows, head_groups), dim3(kF8MergeThreads), 0, s>>>(a);
    if (int rc = check_launch("merge fp8 kernel")) return rc;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_decode_attention_fp8(const pkv_cache8* cache, int32_t layer, void* out, const void* q,
                                        const int32_t* block_tables, int32_t bt_stride, const int32_t* context_lens,
                                        int32_t num_rows, int32_t max_context_len, float scale, void* workspace,
                                        size_t workspace_bytes, void* stream) {
  return pkv::decode_fp8_launch(cache, layer, out, q, nullptr, nullptr, block_tables, bt_stride, context_lens,
                                num_rows, max_context_len, scale, workspace, workspace_bytes, stream);
}

extern "C" int pkv_decode_attention_append_fp8(const pkv_cache8* cache, int32_t layer, void* out, const void* q,
                                               const void* k_new, const void* v_new, const int32_t* block_tables,
                                               int32_t bt_stride, const int32_t* context_lens, int32_t num_rows,
                                               int32_t max_context_len, float scale, void* workspace,
                                               size_t workspace_bytes, void* stream) {
  using namespace pkv;
  if (!k_new || !v_new) return fail(PKV_ERR_INVALID_ARG, "null device pointer");
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return fail(PKV_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  return decode_fp8_launch(cache, layer, out, q, k_new, v_new, block_tables, bt_stride, context_lens, num_rows,
                           max_context_len, scale, workspace, workspace_bytes, stream);
}
