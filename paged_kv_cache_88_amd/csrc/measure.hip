// Measurement kernels: the practical ceilings the decode and prefill kernels are compared against.
//
// read_chunks_kernel reads a buffer as chunks of chunk_bytes taken in a scrambled order, the access pattern of
// the paged decode (a decode unit streams whole (block, kv head) slabs: 4 KB at block size 16, 64 KB at block
// size 256, at addresses its block table scatters over the pool). Decode is bound by these reads (Mini-SGLang
// 源码解析（二）, section 8.3: decode is limited by reading the KV cache), so their sustained rate is the
// ceiling a decode kernel can reach on this GPU, below the published HBM peak.
// mfma_rate_kernel issues independent v_mfma_f32_16x16x32_bf16 chains from every wave: the rate at which the
// matrix cores execute the instruction the prefill kernel is built on, with no memory traffic (prefill is
// bound by compute, same section).
#include "device_common.h"

#include "../../include/pagedkv_measure.h"

namespace pkv {

constexpr int READ_WG = 256;          // 4 waves
constexpr int READ_LOADS = 16;        // 16-byte loads per lane in flight per round (16 KB per wave)

// Wave w of W reads chunks w, w + W, ...; chunk c lives at slot (c * 0x9E3779B1) mod nchunks (nchunks a power
// of two: the odd multiplier makes this a permutation, so every chunk is read once, in scrambled order). A
// chunk is a run of 1 KB pieces (one 16-byte load per lane); a round issues READ_LOADS pieces of the wave's
// list before it consumes any, so 16 KB per wave are in flight (four 4 KB chunks, or a quarter of a 64 KB one).
// Lanes XOR what they load; the result is stored only if it equals a value no buffer here holds, so the loads
// cannot be dropped and the kernel writes nothing in practice.
__global__ void __launch_bounds__(READ_WG)
read_chunks_kernel(const u32x4 *__restrict__ buf, int64_t nchunks, int log2_pieces, u32x4 *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (READ_WG / 64) + (threadIdx.x >> 6);
    const int64_t waves = (int64_t)gridDim.x * (READ_WG / 64);
    const int64_t mine = nchunks > wave ? (nchunks - wave + waves - 1) / waves : 0;   // chunks of this wave
    const int64_t pieces = mine << log2_pieces;
    const int pmask = (1 << log2_pieces) - 1;
    u32x4 acc = {0, 0, 0, 0};
    for (int64_t g0 = 0; g0 < pieces; g0 += READ_LOADS) {
        u32x4 v[READ_LOADS];
#pragma unroll
        for (int u = 0; u < READ_LOADS; ++u) {
            const int64_t g = g0 + u;
            const int64_t c = wave + (g >> log2_pieces) * waves;
            const int64_t slot = (int64_t)(((uint64_t)c * 0x9E3779B1ull) & (uint64_t)(nchunks - 1));
            const int64_t word = ((slot << log2_pieces) + (g & pmask)) * 64 + lane;
            v[u] = g < pieces ? __builtin_nontemporal_load(buf + word) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < READ_LOADS; ++u) acc ^= v[u];
    }
    if (acc[0] == 0x9E3779B1u && acc[1] == 0x7F4A7C15u && acc[2] == 0x85EBCA6Bu && acc[3] == 0xC2B2AE35u)
        sink[(int64_t)blockIdx.x * READ_WG + threadIdx.x] = acc;
}

// Each wave runs CHAINS independent accumulators through `iters` rounds of one MFMA each; operands come from
// the wave's registers (seeded from the lane id), so no memory is touched in the loop.
constexpr int MFMA_CHAINS = 8;

__global__ void __launch_bounds__(256)
mfma_rate_kernel(int iters, f32x4 *__restrict__ sink) {
    const uint32_t lane = threadIdx.x & 63;
    u32x4 a = {0x3f803f80u ^ lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
    u32x4 b = {0x3c003c00u, 0x3c003c00u ^ lane, 0x3c003c00u, 0x3c003c00u};
    f32x4 acc[MFMA_CHAINS];
#pragma unroll
    for (int k = 0; k < MFMA_CHAINS; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < MFMA_CHAINS; ++k) acc[k] = mfma16x16x32(a, b, acc[k]);
    }
    f32x4 s = acc[0];
#pragma unroll
    for (int k = 1; k < MFMA_CHAINS; ++k) s += acc[k];
    if (s[0] == -1.0f && s[1] == -2.0f) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace pkv

extern "C" {

pkv_status pkv_measure_read_chunks(const void *buffer, size_t buffer_bytes, int32_t chunk_bytes, int32_t waves_per_cu,
                                   void *sink, size_t sink_bytes, hipStream_t stream) {
    if (!buffer || !sink || chunk_bytes < 1024 || (chunk_bytes & (chunk_bytes - 1)) || waves_per_cu < 4 ||
        waves_per_cu % 4 || waves_per_cu > 32 || ((uintptr_t)buffer & 15u) || ((uintptr_t)sink & 15u))
        return PKV_EINVAL;
    int64_t nchunks = (int64_t)(buffer_bytes / (size_t)chunk_bytes);
    if (nchunks < 1) return PKV_EINVAL;
    while (nchunks & (nchunks - 1)) nchunks &= nchunks - 1;          // largest power of two that fits
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return PKV_EHIP;
    const int grid = cus * waves_per_cu / 4;
    if (sink_bytes < (size_t)grid * pkv::READ_WG * 16) return PKV_EINVAL;
    int log2_pieces = 0;
    while ((1024 << log2_pieces) < chunk_bytes) ++log2_pieces;
    hipLaunchKernelGGL(pkv::read_chunks_kernel, dim3(grid), dim3(pkv::READ_WG), 0, stream,
                       (const pkv::u32x4 *)buffer, nchunks, log2_pieces, (pkv::u32x4 *)sink);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

int64_t pkv_measure_read_chunks_bytes(size_t buffer_bytes, int32_t chunk_bytes) {
    if (chunk_bytes < 1) return 0;
    int64_t nchunks = (int64_t)(buffer_bytes / (size_t)chunk_bytes);
    if (nchunks < 1) return 0;
    while (nchunks & (nchunks - 1)) nchunks &= nchunks - 1;
    return nchunks * chunk_bytes;
}

pkv_status pkv_measure_mfma_rate(int32_t iters, int32_t waves_per_cu, void *sink, size_t sink_bytes,
                                 double *flops, hipStream_t stream) {
    if (!sink || !flops || iters < 1 || waves_per_cu < 4 || waves_per_cu % 4 || waves_per_cu > 32 ||
        ((uintptr_t)sink & 15u))
        return PKV_EINVAL;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return PKV_EHIP;
    const int grid = cus * waves_per_cu / 4;
    if (sink_bytes < (size_t)grid * 256 * 16) return PKV_EINVAL;
    *flops = (double)grid * 4 * iters * pkv::MFMA_CHAINS * (16.0 * 16.0 * 32.0 * 2.0);
    hipLaunchKernelGGL(pkv::mfma_rate_kernel, dim3(grid), dim3(256), 0, stream, iters, (pkv::f32x4 *)sink);
    return hipGetLastError() == hipSuccess ? PKV_OK : PKV_EHIP;
}

}  // extern "C"
