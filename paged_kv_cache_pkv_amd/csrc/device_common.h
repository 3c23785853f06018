// Device-side helpers for the gfx950 kernels: FP16 vector types, wave64 lane
// shuffles via DPP, and the validation shared by the launch wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "pkv.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kHeadDim = 128;
constexpr int kBlockSize = 16;
constexpr float kLog2e = 1.4426950408889634f;
// Running-max seed: finite, so that exp2(m_old - m_new) stays 1 (not NaN)
// while a lane has seen only masked keys.
constexpr float kMinusBig = -1.0e30f;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& v) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, v);
}

// DPP lane moves within a row of 16 lanes (bound_ctrl on, all rows/banks).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return bitcast<float>(__builtin_amdgcn_mov_dpp(bitcast<int>(v), kCtrl, 0xF, 0xF, true));
}

// Sum over each aligned group of 16 lanes; every lane of the group receives
// the same bits (each step adds a pair in both orders, which IEEE addition
// makes identical).
__device__ __forceinline__ float sum16(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dpp_mov<0x141>(v);  // row_half_mirror: quad 0 <-> quad 1, quad 2 <-> quad 3
  v += dpp_mov<0x140>(v);  // row_mirror: half-row 0 <-> half-row 1
  return v;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  const int lane = __lane_id();
  return bitcast<float>(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, bitcast<int>(v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Dot product of 8 FP16 pairs accumulated in fp32 (v_dot2_f32_f16; the
// products of FP16 values are exact in fp32).
__device__ __forceinline__ float dot8(const uint4& a, const uint4& b) {
  float acc = 0.0f;
  acc = __builtin_amdgcn_fdot2(bitcast<half2_t>(a.x), bitcast<half2_t>(b.x), acc, false);
  acc = __builtin_amdgcn_fdot2(bitcast<half2_t>(a.y), bitcast<half2_t>(b.y), acc, false);
  acc = __builtin_amdgcn_fdot2(bitcast<half2_t>(a.z), bitcast<half2_t>(b.z), acc, false);
  acc = __builtin_amdgcn_fdot2(bitcast<half2_t>(a.w), bitcast<half2_t>(b.w), acc, false);
  return acc;
}

__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
  const half2_t a = bitcast<half2_t>(v.x), b = bitcast<half2_t>(v.y);
  const half2_t c = bitcast<half2_t>(v.z), d = bitcast<half2_t>(v.w);
  f[0] = (float)a.x; f[1] = (float)a.y; f[2] = (float)b.x; f[3] = (float)b.y;
  f[4] = (float)c.x; f[5] = (float)c.y; f[6] = (float)d.x; f[7] = (float)d.y;
}

// fp32 -> FP16 with round-to-nearest-even, packed two per word.
__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  half2_t h;
  h.x = (_Float16)lo;
  h.y = (_Float16)hi;
  return bitcast<uint32_t>(h);
}

// Element offset (in FP16 units) of pool[block][layer][kv][head][0][0].
__device__ __forceinline__ size_t slab_offset(int block, int layer, int kv, int head, int num_layers, int num_heads) {
  return ((((size_t)block * num_layers + layer) * 2 + kv) * num_heads + head) * (size_t)(kBlockSize * kHeadDim);
}

// ---------------------------------------------------------------- host side

inline int check_cache(const pkv_cache* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARG, "cache is null");
  if (!c->base) return fail(PKV_ERR_INVALID_ARG, "cache->base is null");
  if (c->block_size != kBlockSize) return fail(PKV_ERR_UNSUPPORTED, "only block_size 16 is supported");
  if (c->head_dim != kHeadDim) return fail(PKV_ERR_UNSUPPORTED, "only head_dim 128 is supported");
  if (c->num_heads < 1 || c->num_heads > 128) return fail(PKV_ERR_UNSUPPORTED, "num_heads must be in [1, 128]");
  if (c->num_blocks < 1 || c->num_layers < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks and num_layers must be >= 1");
  return PKV_OK;
}

inline int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  clear_error();
  return PKV_OK;
}

inline size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

}  // namespace pkv
