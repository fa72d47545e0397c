// paged_attention_prefill: varlen chunked prefill over the paged cache, on MFMA.
//
// What is computed: sequence i owns query rows [cu_q[i], cu_q[i+1]) (Lq of them) and has
// Lk = cu_k[i+1] - cu_k[i] tokens in the cache, the chunk being the last Lq; P = Lk - Lq is the cached
// prefix. Query row j (position P + j) attends, when causal, to logical tokens [0, P + j], else to
// [0, Lk); keys are read through the block table exactly as in decode.
// (nano-vllm walkthrough, section 2 context: cu_seqlens_q/k, max_seqlen_q/k, block_tables;
// Mini-SGLang 源码解析（二）, sections 6.6 and 6.9: a chunk extends the cached length, chunks of a
// long prompt are fed one after another; "推理运行时", section Prefill 与 decode 输入: tokens of all
// requests are flattened with per-sequence query ranges, and chunked prefill has a cached history.)
// Prefill is bound by compute (Mini-SGLang 源码解析（二）, section 8.3), so both products run on
// MFMA: v_mfma_f32_16x16x32_bf16, bf16 operands, fp32 accumulation.
//
// Work decomposition. Grid (query tile, kv head, sequence). A 256-thread workgroup (4 waves) owns
// 128 "rows" = BQ query positions x the G query heads that share the kv head (row = pos * G + h),
// so each K/V tile brought into LDS serves all G heads. Each wave owns 32 rows (two 16-row MFMA
// blocks). The key loop walks 64-key tiles up to the last key any row of the tile may see:
//   1. the workgroup gathers the tile's K rows (row-major) and V rows (transposed, key-contiguous)
//      from their physical blocks into LDS;
//   2. S = Q K^T on MFMA (Q stays in registers as the A operand);
//   3. mask (causal, bottom-right aligned, and the sequence end), online softmax per row in log2
//      units with a 16-lane DPP max; P is rounded to bf16 and staged in LDS to become an A operand;
//   4. O += P V on MFMA with V^T from LDS as the B operand.
// The MFMA output layout is the 16x16 fp32 block with lane l holding rows 4*(l/16)+i, column l%16;
// the A/B operands take 8 consecutive bf16 of the reduction index per lane, the same rule for both
// operands, so any reduction order the hardware uses pairs matching elements.
#include "device_common.h"
#include "launch.h"

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int PF_THREADS = 256;
constexpr int PF_D = 128;
constexpr int PF_BN = 64;                 // keys per tile
constexpr int PF_ROWS = 128;              // rows per workgroup
constexpr int PF_WROWS = 32;              // rows per wave
constexpr int PF_KPAD = PF_D + 8;         // LDS row stride of K, bf16 elements (272 bytes)
constexpr int PF_VPAD = PF_BN + 8;        // LDS row stride of V^T (144 bytes)
constexpr int PF_PPAD = PF_BN + 8;        // LDS row stride of P (144 bytes)
constexpr float PF_M_INIT = -1.0e30f;

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dppf<DPP_XOR1>(v));
    v = fmaxf(v, dppf<DPP_XOR2>(v));
    v = fmaxf(v, dppf<DPP_HALF_MIRROR>(v));
    v = fmaxf(v, dppf<DPP_MIRROR>(v));
    return v;
}

template <int G>
__global__ void __launch_bounds__(PF_THREADS)
prefill_kernel(uint16_t *__restrict__ out, const u32x4 *__restrict__ query, const u32x4 *__restrict__ key_cache,
               const u32x4 *__restrict__ value_cache, const int32_t *__restrict__ block_tables, int bt_stride,
               const int32_t *__restrict__ cu_seqlens_q, const int32_t *__restrict__ cu_seqlens_k, int max_seqlen_k,
               int num_kv_heads, int64_t num_blocks, int log2_bs, float scale_log2e, int causal) {
    constexpr int BQ = PF_ROWS / G;           // query positions per workgroup
    constexpr int VR = BQ * G;                // rows in use (<= 128)
    constexpr int CH = PF_D / 8;              // 16-byte chunks per K/V row

    __shared__ __attribute__((aligned(16))) uint16_t sK[PF_BN * PF_KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t sV[PF_D * PF_VPAD];
    __shared__ __attribute__((aligned(16))) uint16_t sP[PF_THREADS / 64][PF_WROWS * PF_PPAD];

    const int qt = blockIdx.x, kvh = blockIdx.y, seq = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lr = lane & 15, lb = lane >> 4;       // MFMA lane row / lane block
    const int num_heads = num_kv_heads * G;

    const int q0 = cu_seqlens_q[seq];
    const int Lq = cu_seqlens_q[seq + 1] - q0;
    const int Lk = min(cu_seqlens_k[seq + 1] - cu_seqlens_k[seq], max_seqlen_k);
    const int P = Lk - Lq;
    const int pos0 = qt * BQ;
    if (Lq <= 0 || P < 0 || pos0 >= Lq) return;
    const int npos = min(BQ, Lq - pos0);
    const int kend = causal ? min(Lk, P + pos0 + npos) : Lk;   // keys [0, kend) may be visible
    const int ntiles = (kend + PF_BN - 1) / PF_BN;
    const int bs_mask = (1 << log2_bs) - 1;
    const int32_t *bt = block_tables + (int64_t)seq * bt_stride;

    // Q operand: this lane supplies row (wave*32 + rb*16 + lr), dims 8*lb + 32*ks .. +8
    u32x4 qa[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int r = wave * PF_WROWS + rb * 16 + lr;
        const int pos = r / G, h = r % G;
        const bool ok = r < VR && pos < npos;
        const int64_t qrow = ((int64_t)(q0 + pos0 + (ok ? pos : 0)) * num_heads + kvh * G + h) * CH;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qa[rb][ks] = ok ? query[qrow + lb + 4 * ks] : u32x4{0, 0, 0, 0};
    }

    f32x4 o[2][8];
    float m[2][4], l[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int db = 0; db < 8; ++db) o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            m[rb][i] = PF_M_INIT;
            l[rb][i] = 0.f;
        }
    }

    for (int kt = 0; kt < ntiles; ++kt) {
        const int key0 = kt * PF_BN;
        // 1. gather the tile: 64 keys x 16 chunks; K row-major, V transposed
#pragma unroll
        for (int c = 0; c < (PF_BN * CH) / PF_THREADS; ++c) {
            const int idx = tid + c * PF_THREADS;
            const int key = idx / CH, ch = idx % CH;
            const int gk = key0 + key;
            u32x4 kv = u32x4{0, 0, 0, 0}, vv = u32x4{0, 0, 0, 0};
            if (gk < kend) {
                const int64_t blk = bt[gk >> log2_bs];
                if (blk >= 0 && blk < num_blocks) {
                    const int64_t row = ((blk * num_kv_heads + kvh) << log2_bs) + (gk & bs_mask);
                    kv = key_cache[row * CH + ch];
                    vv = value_cache[row * CH + ch];
                }
            }
            *(u32x4 *)&sK[key * PF_KPAD + ch * 8] = kv;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sV[(ch * 8 + 2 * j) * PF_VPAD + key] = (uint16_t)(vv[j] & 0xffffu);
                sV[(ch * 8 + 2 * j + 1) * PF_VPAD + key] = (uint16_t)(vv[j] >> 16);
            }
        }
        __syncthreads();

        // 2. S = Q K^T for this wave's 32 rows x 64 keys
        f32x4 s[2][4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            s[0][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
            s[1][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const u32x4 kb = *(const u32x4 *)&sK[(nb * 16 + lr) * PF_KPAD + lb * 8 + ks * 32];
                s[0][nb] = mfma16x16x32(qa[0][ks], kb, s[0][nb]);
                s[1][nb] = mfma16x16x32(qa[1][ks], kb, s[1][nb]);
            }
        }

        // 3. mask, online softmax, P -> LDS (bf16)
        uint16_t *pw = sP[wave];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wave * PF_WROWS + rb * 16 + lb * 4 + i;
                const int pos = r / G;
                const bool row_ok = r < VR && pos < npos;
                const int kmax = causal ? P + pos0 + pos : Lk - 1;     // last visible key
                float mx = -INFINITY;
                float sv[4];
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int key = key0 + nb * 16 + lr;
                    const bool ok = row_ok && key < kend && key <= kmax;
                    sv[nb] = ok ? s[rb][nb][i] * scale_log2e : -INFINITY;
                    mx = fmaxf(mx, sv[nb]);
                }
                mx = row16_max(mx);
                const float m_new = fmaxf(m[rb][i], mx);
                const float alpha = fast_exp2(m[rb][i] - m_new);
                m[rb][i] = m_new;
                float rs = 0.f;
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const float p = fast_exp2(sv[nb] - m_new);
                    const uint32_t pb = f32_to_bf16_rne(p);
                    rs += __uint_as_float(pb << 16);        // sum the rounded weights the MFMA uses
                    pw[(rb * 16 + lb * 4 + i) * PF_PPAD + nb * 16 + lr] = (uint16_t)pb;
                }
                l[rb][i] = l[rb][i] * alpha + rs;
#pragma unroll
                for (int db = 0; db < 8; ++db) o[rb][db][i] *= alpha;
            }
        }
        __syncthreads();

        // 4. O += P V
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            const u32x4 pa0 = *(const u32x4 *)&pw[(0 * 16 + lr) * PF_PPAD + lb * 8 + ks * 32];
            const u32x4 pa1 = *(const u32x4 *)&pw[(1 * 16 + lr) * PF_PPAD + lb * 8 + ks * 32];
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const u32x4 vb = *(const u32x4 *)&sV[(db * 16 + lr) * PF_VPAD + lb * 8 + ks * 32];
                o[0][db] = mfma16x16x32(pa0, vb, o[0][db]);
                o[1][db] = mfma16x16x32(pa1, vb, o[1][db]);
            }
        }
        __syncthreads();
    }

    // normalise and write: lane holds rows 4*lb + i of each 16-row block, column lr of each 16-dim block
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lsum = group_sum<16>(l[rb][i]);
            const int r = wave * PF_WROWS + rb * 16 + lb * 4 + i;
            const int pos = r / G, h = r % G;
            if (r >= VR || pos >= npos) continue;
            const float inv = 1.0f / lsum;
            uint16_t *orow = out + ((int64_t)(q0 + pos0 + pos) * num_heads + kvh * G + h) * PF_D;
#pragma unroll
            for (int db = 0; db < 8; ++db) orow[db * 16 + lr] = (uint16_t)f32_to_bf16_rne(o[rb][db][i] * inv);
        }
    }
}

template <int G>
static hipError_t launch_prefill_g(const PrefillArgs &a, hipStream_t stream) {
    constexpr int BQ = PF_ROWS / G;
    dim3 grid((a.max_seqlen_q + BQ - 1) / BQ, a.num_kv_heads, a.num_seqs);
    hipLaunchKernelGGL((prefill_kernel<G>), grid, dim3(PF_THREADS), 0, stream, (uint16_t *)a.out,
                       (const u32x4 *)a.query, (const u32x4 *)a.key_cache, (const u32x4 *)a.value_cache, a.block_tables,
                       a.bt_stride, a.cu_seqlens_q, a.cu_seqlens_k, a.max_seqlen_k, a.num_kv_heads, a.num_blocks,
                       a.log2_bs, a.scale_log2e, a.causal);
    return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, bool bf16, int head_dim, int group, hipStream_t stream) {
    if (!bf16 || head_dim != PF_D) return hipErrorInvalidValue;
    if (a.num_seqs == 0 || a.max_seqlen_q == 0) return hipSuccess;
    switch (group) {
        case 1: return launch_prefill_g<1>(a, stream);
        case 2: return launch_prefill_g<2>(a, stream);
        case 3: return launch_prefill_g<3>(a, stream);
        case 4: return launch_prefill_g<4>(a, stream);
        case 5: return launch_prefill_g<5>(a, stream);
        case 6: return launch_prefill_g<6>(a, stream);
        case 7: return launch_prefill_g<7>(a, stream);
        case 8: return launch_prefill_g<8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pkv
