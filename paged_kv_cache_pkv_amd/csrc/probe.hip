// Bandwidth and matrix-core probes (measurement aid; see pkv_probe.h).
// Loads are 16-byte buffer loads, eight in flight per lane, through buffer
// resources whose range check turns any offset past the region into a zero
// read.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkv_probe.h"

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;
constexpr uint32_t kMagic = 0x9E3779B9u;  // the sink is written only if a lane's fold equals this

template <int kCpol>
__device__ __forceinline__ uint32_t fold_loads(__amdgpu_buffer_rsrc_t rs, uint32_t first, uint32_t step,
                                               uint32_t end) {
  uint32_t acc = 0;
  for (uint32_t o = first; o < end; o += step * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, o + u * step, 0, kCpol));
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  return acc;
}

template <int kCpol>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const char* src, uint32_t nbytes, uint32_t* sink) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(src), 0, nbytes, 0x00020000);
  const uint32_t step = gridDim.x * kThreads * 16u;
  const uint32_t acc = fold_loads<kCpol>(rs, (blockIdx.x * kThreads + threadIdx.x) * 16u, step, nbytes);
  if (acc == kMagic) sink[0] = acc;
}

template <int kCpol>
__global__ __launch_bounds__(kThreads) void slab_read_kernel(const char* base, size_t base_bytes,
                                                             const int32_t* slab_index, uint32_t slab_bytes,
                                                             uint32_t* sink) {
  const int32_t idx = slab_index[blockIdx.x];
  const size_t off = (size_t)(idx < 0 ? 0 : idx) * slab_bytes;
  if (idx < 0 || off + slab_bytes > base_bytes) return;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + off), 0, slab_bytes, 0x00020000);
  const uint32_t acc = fold_loads<kCpol>(rs, threadIdx.x * 16u, kThreads * 16u, slab_bytes);
  if (acc == kMagic) sink[0] = acc;
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f16v __attribute__((ext_vector_type(16)));

// Four independent accumulation chains per wave keep the matrix core busy
// without any dependency stall; the operands depend on the lane, so nothing
// folds at compile time.
__global__ __launch_bounds__(kThreads) void mfma_f16_kernel(int32_t iters, uint32_t* sink) {
  h8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)((threadIdx.x & 63) * 0.0078125f);
    b[i] = (_Float16)(i * 0.125f - 0.5f);
  }
  f16v c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int32_t i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, a, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(b, b, c3, 0, 0, 0);
  }
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc += (c0[i] + c1[i]) + (c2[i] + c3[i]);
  if (__float_as_uint(acc) == kMagic) sink[0] = kMagic;
}

int launched() { return hipGetLastError() == hipSuccess ? 0 : -7; }

int compute_units(int& cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess)
    return -7;
  if (cus < 1) cus = 256;
  return 0;
}

}  // namespace

extern "C" int pkv_probe_stream_read(const void* src, size_t nbytes, uint32_t* sink, int nontemporal, void* stream) {
  if (!src || !sink || nbytes == 0 || nbytes % 16 || nbytes >= (size_t(1) << 31) ||
      (reinterpret_cast<uintptr_t>(src) & 15))
    return -1;
  int cus = 0;
  if (int rc = compute_units(cus)) return rc;
  const uint32_t per_wg = kThreads * 16u * kUnroll;
  uint32_t grid = (uint32_t)((nbytes + per_wg - 1) / per_wg);
  const uint32_t cap = (uint32_t)cus * 16u;  // enough workgroups to fill every CU
  grid = grid < cap ? grid : cap;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    stream_read_kernel<2><<<grid, kThreads, 0, s>>>(static_cast<const char*>(src), (uint32_t)nbytes, sink);
  else
    stream_read_kernel<0><<<grid, kThreads, 0, s>>>(static_cast<const char*>(src), (uint32_t)nbytes, sink);
  return launched();
}

extern "C" int pkv_probe_slab_read(const void* base, size_t base_bytes, const int32_t* slab_index, int32_t n,
                                   size_t slab_bytes, uint32_t* sink, int nontemporal, void* stream) {
  if (!base || !slab_index || !sink || n < 0 || slab_bytes == 0 || slab_bytes % 4096 ||
      slab_bytes >= (size_t(1) << 31) || (reinterpret_cast<uintptr_t>(base) & 15))
    return -1;
  if (n == 0) return 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nontemporal)
    slab_read_kernel<2><<<n, kThreads, 0, s>>>(static_cast<const char*>(base), base_bytes, slab_index,
                                               (uint32_t)slab_bytes, sink);
  else
    slab_read_kernel<0><<<n, kThreads, 0, s>>>(static_cast<const char*>(base), base_bytes, slab_index,
                                               (uint32_t)slab_bytes, sink);
  return launched();
}

extern "C" int pkv_probe_mfma_f16(int32_t iters, uint32_t* sink, double* flops, void* stream) {
  if (!sink || !flops || iters < 1 || iters > (1 << 24)) return -1;
  int cus = 0;
  if (int rc = compute_units(cus)) return rc;
  const uint32_t grid = (uint32_t)cus * 4u;
  *flops = (double)grid * (kThreads / 64) * (double)iters * 4.0 * (2.0 * 32 * 32 * 16);
  mfma_f16_kernel<<<grid, kThreads, 0, static_cast<hipStream_t>(stream)>>>(iters, sink);
  return launched();
}
