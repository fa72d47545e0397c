/*
 * pagedkv_measure.h -- measurement entry points of libpagedkv.so: the practical ceilings that the decode
 * and prefill kernels are reported against, beside the GPU's published peaks. They compute nothing of the
 * paged cache itself.
 *
 * Decode is bound by reading the KV cache and prefill by compute (Mini-SGLang 源码解析（二）, section 8.3).
 * A decode unit streams whole (block, kv head) slabs of its sequence (block_size x head_dim elements: 4 KB
 * at block size 16 and 64 KB at block size 256 in bf16 at head_dim 128) from wherever its block table
 * points ("推理运行时", section 分页 KV); the prefill kernel's products are v_mfma_f32_16x16x32_bf16.
 *
 * Ownership, ordering and errors as in pagedkv.h: device pointers, nothing allocated, calls enqueued on
 * `stream`; PKV_EINVAL for bad arguments (nothing launched), PKV_EHIP for launch failures.
 */
#ifndef PAGEDKV_MEASURE_H
#define PAGEDKV_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * measure_read_chunks: read the first pkv_measure_read_chunks_bytes(buffer_bytes, chunk_bytes) bytes of
 * `buffer` (device, 16-byte aligned) once, as chunks of chunk_bytes (a power of two, >= 1024) visited in a
 * scrambled order (chunk c at slot c * 0x9E3779B1 mod the chunk count, a power of two), with 16-byte
 * non-temporal loads from waves_per_cu waves per compute unit (4..32, a multiple of 4), each keeping 16 KB of
 * its chunks in flight. Time it with events
 * on `stream`: bytes / time is the sustained rate of the decode's access pattern. `sink` (device, 16-byte
 * aligned, sink_bytes >= 4096 * compute units * waves_per_cu / 4) is written only in the impossible case that
 * the XOR of the data read equals a fixed 128-bit value; it keeps the loads from being optimised away.
 */
pkv_status pkv_measure_read_chunks(const void *buffer, size_t buffer_bytes, int32_t chunk_bytes, int32_t waves_per_cu,
                                   void *sink, size_t sink_bytes, hipStream_t stream);

/* Bytes one pkv_measure_read_chunks call reads: the largest power-of-two count of whole chunks that fits. */
int64_t pkv_measure_read_chunks_bytes(size_t buffer_bytes, int32_t chunk_bytes);

/*
 * measure_mfma_rate: every wave of waves_per_cu per compute unit (4..32, a multiple of 4) runs `iters` rounds
 * of 8 independent v_mfma_f32_16x16x32_bf16 on register operands (no memory traffic). *flops (host) receives
 * the launch's flop count (2 * 16 * 16 * 32 per instruction); flops / time is the rate the matrix cores
 * sustain for that instruction. `sink` (device, 16-byte aligned, sink_bytes >= 4096 * compute units *
 * waves_per_cu / 4) is written only if the sums take values they cannot take.
 */
pkv_status pkv_measure_mfma_rate(int32_t iters, int32_t waves_per_cu, void *sink, size_t sink_bytes, double *flops,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_MEASURE_H */
