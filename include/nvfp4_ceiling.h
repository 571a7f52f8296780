/*
 * nvfp4_ceiling.h -- C ABI of libnvfp4_ceiling.so, the measurement kernels
 * the benchmark times beside the NVFP4 kernels to state what this GPU allows
 * (they are not part of the NVFP4 path and share no code with it).
 *
 * Every call enqueues one kernel on `stream` and returns 0 (hipSuccess) or a
 * hipError_t code; arguments are checked before anything is enqueued
 * (hipErrorInvalidValue).  Pointers are device pointers owned by the caller.
 */
#ifndef NVFP4_CEILING_H
#define NVFP4_CEILING_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * nvfp4_ceiling_read -- read `bytes` (a positive multiple of 16) of device
 * memory at p once with 16-byte nontemporal loads, all of a thread's eight
 * loads issued before any use; the data is folded into a word that is
 * practically never stored to sink (one device uint32).
 */
int nvfp4_ceiling_read(const void* p, uint64_t bytes, uint32_t* sink, hipStream_t stream);

/*
 * nvfp4_ceiling_copy -- copy `bytes` (a positive multiple of 16) from src to
 * dst with the loads of nvfp4_ceiling_read and 16-byte stores.
 */
int nvfp4_ceiling_copy(const void* src, void* dst, uint64_t bytes, hipStream_t stream);

/*
 * nvfp4_ceiling_mfma -- `blocks` workgroups of 4 waves, each wave running
 * iters x 4 v_mfma_f32_32x32x16_bf16 (32768 flop each) on four independent
 * accumulators with no memory traffic.  clocks (two device uint64) receives,
 * for wave 0 of workgroup 0, the shader-clock cycles (s_memtime) and the
 * 100 MHz real-time ticks (s_memrealtime) its loop took; their ratio times
 * 100 MHz is the shader clock during the loop.  sink: one device float,
 * practically never written.
 */
int nvfp4_ceiling_mfma(int64_t iters, int blocks, float* sink, uint64_t* clocks,
                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_CEILING_H */
