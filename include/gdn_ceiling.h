/*
 * gdn_ceiling.h — measurement kernels of libgdn_ceiling.so: the achievable HBM and
 * MFMA rates of the GPU the layer runs on, against which the layer's kernels are
 * reported next to the datasheet peaks. The mlxcel benchmark notes
 * (lablup/mlxcel docs/benchmarks.md, the run-record list and the pipelined-timing
 * section) ask for measured ceilings beside every roofline figure; these kernels are
 * that measurement and are not part of the layer (include/gdn.h).
 *
 * Conventions: device pointers, 16-byte aligned; `bytes` a multiple of 64; `grid`
 * workgroups of 256 threads (1 .. 2^20); `stream` a hipStream_t (NULL = default). Each
 * call validates its arguments (returning 1 and launching nothing on a bad argument),
 * enqueues one kernel and returns 0, or 2 when the launch fails. Nothing synchronises.
 */
#ifndef GDN_CEILING_H_
#define GDN_CEILING_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` from src with 16-byte loads (grid-stride); sink [grid] receives one
 * value per workgroup only in a case that never happens with finite data, so it stays
 * unwritten in practice but keeps the loads. */
int gdn_ceiling_read(const void* src, size_t bytes, float* sink, int grid, void* stream);

/* Writes `bytes` of zeros to dst with 16-byte stores; nontemporal != 0 uses streaming
 * (non-temporal) stores, as the layer's state stores do. */
int gdn_ceiling_write(void* dst, size_t bytes, int nontemporal, int grid, void* stream);

/* Copies `bytes` from src to dst (must not overlap) with 16-byte loads and stores. */
int gdn_ceiling_copy(const void* src, void* dst, size_t bytes, int nontemporal, int grid,
                     void* stream);

/* Blocked forms of the three: workgroup b (256 threads) moves the contiguous block of
 * per_thread * 4096 bytes at offset b * per_thread * 4096, a thread's per_thread 16-byte
 * granules 4096 bytes apart, all its loads issued before any of its stores (the access
 * pattern of the layer's commit kernel). per_thread is 4, 8 or 16; bytes a multiple of
 * per_thread * 4096 and at most 2^20 blocks; the grid is bytes / (per_thread * 4096). */
int gdn_ceiling_read_blocked(const void* src, size_t bytes, float* sink, int per_thread, void* stream);
int gdn_ceiling_write_blocked(void* dst, size_t bytes, int nontemporal, int per_thread, void* stream);
int gdn_ceiling_copy_blocked(const void* src, void* dst, size_t bytes, int nontemporal, int per_thread,
                             void* stream);

/* `iters` rounds of 8 independent MFMA products per wave, 4 waves per workgroup. dtype
 * 0: v_mfma_f32_16x16x32_f16, 1: ..._16x16x32_bf16 (16384 flops each: grid * 4 * iters *
 * 8 * 16384 in all); 2: v_mfma_f32_32x32x16_f16, 3: ..._32x32x16_bf16 (32768 flops each).
 * sink [grid] as for gdn_ceiling_read. */
int gdn_ceiling_mfma(float* sink, int grid, int iters, int dtype, void* stream);

/* Compute units, peak shader clock (kHz), memory clock (kHz) and memory bus width (bits)
 * of HIP device `device`; 0 on success. */
int gdn_ceiling_device_info(int device, int* cus, int* clock_khz, int* mem_clock_khz,
                            int* mem_bus_bits);

#ifdef __cplusplus
}
#endif

#endif /* GDN_CEILING_H_ */
