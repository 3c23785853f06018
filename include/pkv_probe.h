/*
 * pkv_probe.h - bandwidth and matrix-core probes for MI355X (gfx950): a
 * measurement aid built beside libpkv.so into libpkv_probe.so.  Not part of
 * the paged-attention interface in pkv.h; nothing in libpkv.so calls these.
 *
 * They measure the read bandwidth a memory-bound kernel can reach on the box,
 * the ceiling against which the decode kernels' achieved bandwidth is read
 * (Inference Infrastructure, seeitflow.com: after "Three iterations with the
 * state written out", reading the KV cache at the memory bandwidth sets the
 * decode step's floor), and the FP16 matrix-core rate a kernel sustains, the
 * ceiling of the prefill tile's matrix products (The inference engine,
 * wpnews.pro, "Prefill and decode ask the accelerator for different work").
 * Every result feeds a comparison whose store (to sink[0]) essentially never
 * happens, so no load or product can be dropped.
 *
 * Return value: 0, or -1 for an invalid argument (nothing launched), or -7
 * when the HIP runtime refuses the launch.  All pointers are device pointers
 * owned by the caller; calls are asynchronous on `stream` (a hipStream_t, NULL
 * for the default stream).  nontemporal != 0 gives the loads the streaming
 * cache policy the decode kernels use.
 */
#ifndef PKV_PROBE_H
#define PKV_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read bytes [0, nbytes) of src once, 16 bytes per lane and load, grid-stride.
 * nbytes must be a multiple of 16 and below 2^31; src 16-byte aligned. */
int pkv_probe_stream_read(const void* src, size_t nbytes, uint32_t* sink, int nontemporal, void* stream);

/* Read n slabs of slab_bytes each, slab i at byte offset
 * slab_index[i] * slab_bytes of base (a device region of base_bytes bytes),
 * one workgroup per slab.  With the paged pool [blocks][layers][2][heads][16]
 * [128] FP16, a (block, layer) slab is the 2 * heads * 4 KiB of K and V one
 * decode step reads for that block, and slab_index[i] = block * layers +
 * layer.  slab_index is a device int32 array [n]; an index whose slab falls
 * outside base_bytes is skipped.  slab_bytes must be a multiple of 4096 and
 * below 2^31; base 16-byte aligned. */
int pkv_probe_slab_read(const void* base, size_t base_bytes, const int32_t* slab_index, int32_t n, size_t slab_bytes,
                        uint32_t* sink, int nontemporal, void* stream);

/* Sustained FP16 matrix-core rate: 4 workgroups of 4 waves per compute unit,
 * each wave running `iters` rounds of four independent
 * v_mfma_f32_32x32x16_f16 chains (operands in registers, nothing read from
 * memory).  *flops (host pointer) receives the launch's floating-point
 * operations, 2 * 32 * 32 * 16 per product; divide by the launch's time.
 * iters must be in [1, 2^24]. */
int pkv_probe_mfma_f16(int32_t iters, uint32_t* sink, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_PROBE_H */
