// paged_attention_decode: one query token per sequence attends over the context_lens[i] tokens
// that its block table points to (the token stored this step included).
//
// What is computed: for query head h of sequence i, kv head h / G (G = num_heads / num_kv_heads),
//   out = sum_t softmax_t(scale * q . k_t) v_t over logical tokens t < context_lens[i],
// where logical token t lives in physical block block_tables[i][t / block_size] at offset
// t % block_size ("推理运行时", section 分页 KV: the block table maps logical to physical blocks
// and the attention kernel reads K/V through it; "LLM Infra 101 v0.2: KV Cache", section 推理:
// the new token attends to the cached tokens and itself). Decode is bound by reading the cache
// (Mini-SGLang 源码解析（二）, section 8.3), so the kernel is built around streaming K/V once,
// with enough bytes in flight to cover HBM latency.
//
// Work decomposition. A partition is a run of part_tokens logical tokens of one sequence (a multiple
// of block_size, spanning at most 64 blocks). A one-workgroup plan kernel reads context_lens on the
// device and writes the list of (sequence, partition) work items sorted longest first (a counting sort
// on the partition's token count), so long partitions are dispatched first and the batch does not end
// on a straggler. The decode grid is one workgroup per (work item, kv head) in that order; slots past
// the item count exit at once. A workgroup of NW waves serves all G query heads of its kv head, so
// every K/V byte is read once. If a sequence fits one partition the workgroup writes the final output;
// otherwise it writes an unnormalised partial (running max m, sum l, accumulator o, fp32) and the
// reduce kernel merges the partitions with the log-sum-exp rule.
//
// Inside a wave: LPT lanes share one token row (head_dim elements); each lane holds NV 16-byte
// vectors of the row, so one load instruction covers RPW = 64 / LPT rows. A wave tile is R such
// instructions (TILE = R * RPW tokens); tiles are dealt to the NW waves round-robin. Each wave runs a
// two-stage software pipeline: the loads of its next tile are in flight while it computes the current
// one. The partition's block-table slice (<= 64 ids) sits one id per lane in a register and is read
// with a lane shuffle, so the only dependent memory round trip per tile is the K/V load itself.
// Each LPT-lane group keeps its own online-softmax state (m, l, acc) for the G heads; groups, then
// waves, are merged once at the end. For bf16 data both products use v_dot2_f32_bf16: q.k on bf16
// pairs of the row, and p.v on the weights of two rows rounded to a bf16 pair (fp32 FMAs for fp32
// data). The group sum is a DPP butterfly; softmax runs in log2 units (exp2 with scale*log2(e) folded
// in), and the accumulator is rescaled only when some running max of the wave grows.
#include "device_common.h"
#include "launch.h"

namespace pkv {

#ifndef PKV_DECODE_NT
#define PKV_DECODE_NT 1      // K/V loads are marked non-temporal: each byte is streamed once
#endif

constexpr int MAX_PART_BLOCKS = 64;           // block-table entries one partition may span
constexpr float M_INIT = -1.0e30f;            // finite "minus infinity": keeps exp2(m - m') finite

template <bool BF16, int D, int G, int NV_, int R_, int NW_>
struct DecodeShape {
    static constexpr int ES = BF16 ? 2 : 4;                     // element bytes
    static constexpr int VEC = 16 / ES;                         // elements per 16-byte vector
    static constexpr int VPR = D / VEC;                         // vectors per row
    static constexpr int NV = NV_;                              // vectors per lane per row
    static constexpr int LPT = VPR / NV;                        // lanes per token row
    static constexpr int RPW = 64 / LPT;                        // rows per wave instruction
    static constexpr int R = R_;                                // instructions per tile
    static constexpr int TILE = R * RPW;                        // tokens per wave tile
    static constexpr int EPL = NV * VEC;                        // elements per lane
    static constexpr int NW = NW_;                              // waves per workgroup
    static_assert(VPR % NV == 0 && LPT >= 1 && LPT <= 16 && (LPT & (LPT - 1)) == 0, "lanes per token");
    static_assert(!BF16 || R % 2 == 0, "bf16 p.v pairs rows: R must be even");
};

template <class S>
struct TileRegs {
    u32x4 k[S::R][S::NV];
    u32x4 v[S::R][S::NV];
    bool valid[S::R];
};

constexpr int PLAN_THREADS = 1024;
constexpr int PLAN_BUCKETS = 64;

// Work list for the decode grid. items[k] = {seq, part, ntok, nparts}, sorted by ntok descending in
// PLAN_BUCKETS buckets (order inside a bucket is arbitrary: every item writes its own output, so the
// result does not depend on it). ctrl[0] = number of items. Sequences with an empty context get zero
// outputs here. Single workgroup.
__global__ void __launch_bounds__(PLAN_THREADS)
decode_plan_kernel(const int32_t *__restrict__ context_lens, int num_seqs, int max_context_len, int part_tokens,
                   int4 *__restrict__ items, int *__restrict__ ctrl, void *__restrict__ out, int out_row_elems,
                   int elem_bytes) {
    __shared__ int hist[PLAN_BUCKETS];
    __shared__ int offs[PLAN_BUCKETS];
    const int tid = threadIdx.x;
    if (tid < PLAN_BUCKETS) hist[tid] = 0;
    __syncthreads();
    auto bucket = [&](int ntok) { return (int)(((int64_t)(part_tokens - ntok) * PLAN_BUCKETS) / part_tokens); };
    for (int i = tid; i < num_seqs; i += PLAN_THREADS) {
        const int L = min(context_lens[i], max_context_len);
        for (int start = 0; start < L; start += part_tokens) atomicAdd(&hist[bucket(min(part_tokens, L - start))], 1);
    }
    __syncthreads();
    if (tid < 64) {                                   // exclusive scan of the 64 buckets in one wave
        const int h = hist[tid];
        int v = h;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(v, o);
            if (tid >= o) v += u;
        }
        offs[tid] = v - h;
        if (tid == 63) ctrl[0] = v;
    }
    __syncthreads();
    for (int i = tid; i < num_seqs; i += PLAN_THREADS) {
        const int L = min(context_lens[i], max_context_len);
        if (L <= 0) {                                 // empty context: zero outputs for every head
            const int64_t n = (int64_t)out_row_elems * elem_bytes / 4;
            uint32_t *o = (uint32_t *)((char *)out + (int64_t)i * out_row_elems * elem_bytes);
            for (int64_t k = 0; k < n; ++k) o[k] = 0u;
            continue;
        }
        const int nparts = (L + part_tokens - 1) / part_tokens;
        for (int part = 0, start = 0; start < L; ++part, start += part_tokens) {
            const int ntok = min(part_tokens, L - start);
            const int pos = atomicAdd(&offs[bucket(ntok)], 1);
            items[pos] = make_int4(i, part, ntok, nparts);
        }
    }
}

template <bool BF16, int D, int G, int NV_, int R_, int NW_>
__global__ void __launch_bounds__(64 * NW_)
decode_kernel(void *__restrict__ out, const void *__restrict__ query, const u32x4 *__restrict__ key_cache,
              const u32x4 *__restrict__ value_cache, const int32_t *__restrict__ block_tables, int bt_stride,
              const int4 *__restrict__ items, const int *__restrict__ ctrl, int num_kv_heads,
              int64_t num_blocks, int log2_bs, int part_tokens, float scale_log2e,
              float *__restrict__ ws_m, float *__restrict__ ws_l, float *__restrict__ ws_o, int max_parts) {
    using S = DecodeShape<BF16, D, G, NV_, R_, NW_>;
    constexpr int NV = S::NV, LPT = S::LPT, RPW = S::RPW, R = S::R, TILE = S::TILE, EPL = S::EPL, VEC = S::VEC;
    constexpr int NW = S::NW;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane / LPT, sub = lane % LPT;
    const int num_heads = num_kv_heads * G;

    // work item in longest-first order; slots past the list exit
    const int slot = blockIdx.x;
    if (slot >= ctrl[0] * num_kv_heads) return;
    const int4 item = items[slot / num_kv_heads];
    const int kvh = slot % num_kv_heads;
    const int seq = item.x, part = item.y, ntok = item.z, nparts = item.w;
    const bool several = nparts > 1;

    // the partition's block-table slice, one id per lane (partitions never pass the table's stride)
    const int start = part * part_tokens;
    const int first_blk = start >> log2_bs;
    const int nbp = part_tokens >> log2_bs;
    int my_blk = -1;
    if (lane < nbp && first_blk + lane < bt_stride) my_blk = block_tables[(int64_t)seq * bt_stride + first_blk + lane];
    const int bs_mask = (1 << log2_bs) - 1;

    // q for the G heads of this kv head: lane holds elements [(v * LPT + sub) * VEC, +VEC) of each
    u32x4 q[G][NV];
    {
        const u32x4 *qv = (const u32x4 *)query;
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int v = 0; v < NV; ++v)
                q[h][v] = qv[((int64_t)seq * num_heads + kvh * G + h) * S::VPR + v * LPT + sub];
    }

    // issue the loads of one tile (addresses clamped to a valid token; validity kept for masking)
    auto issue = [&](int tile, TileRegs<S> &t) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int tl = tile * TILE + r * RPW + grp;
            const bool in = tl < ntok;
            const int tok = start + (in ? tl : 0);
            const int64_t blk = __shfl(my_blk, (tok >> log2_bs) - first_blk);
            t.valid[r] = in && blk >= 0 && blk < num_blocks;
            const int64_t b = t.valid[r] ? blk : 0;
            const int64_t base = (((b * num_kv_heads + kvh) << log2_bs) + (tok & bs_mask)) * S::VPR + sub;
#pragma unroll
            for (int v = 0; v < NV; ++v) {
#if PKV_DECODE_NT
                t.k[r][v] = __builtin_nontemporal_load(key_cache + base + v * LPT);
                t.v[r][v] = __builtin_nontemporal_load(value_cache + base + v * LPT);
#else
                t.k[r][v] = key_cache[base + v * LPT];
                t.v[r][v] = value_cache[base + v * LPT];
#endif
            }
        }
    };

    float m[G], l[G], acc[G][EPL];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = M_INIT;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
    }

    auto compute = [&](int tile, TileRegs<S> &t) {
        bool any_masked = false;
#pragma unroll
        for (int r = 0; r < R; ++r) any_masked |= !t.valid[r];
        const bool partial = __builtin_amdgcn_ballot_w64(any_masked) != 0;   // wave-uniform
        if (partial) {                                      // zero V of masked tokens (they may hold NaN)
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    if (!t.valid[r]) t.v[r][v] = u32x4{0, 0, 0, 0};
        }
        // partial dot products of all (row, head) pairs first, then the group butterfly one step at a
        // time over all of them: no DPP reads a value written by the instruction just before it
        float s[R][G];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float a = 0.f;
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if constexpr (BF16) a = dot2_bf16(q[h][v][j], t.k[r][v][j], a);
                        else a = fmaf(__uint_as_float(q[h][v][j]), __uint_as_float(t.k[r][v][j]), a);
                    }
                s[r][h] = a;
            }
        group_sum_all<LPT, R * G>(&s[0][0]);
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float a = s[r][h] * scale_log2e;
                s[r][h] = (partial && !t.valid[r]) ? -INFINITY : a;
            }
        float m_new[G];
        bool grow = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float mx = s[0][h];
#pragma unroll
            for (int r = 1; r < R; ++r) mx = fmaxf(mx, s[r][h]);
            m_new[h] = fmaxf(m[h], mx);
            grow |= m_new[h] > m[h];
        }
        if (__builtin_amdgcn_ballot_w64(grow)) {            // rescale only when a running max grew
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float alpha = fast_exp2(m[h] - m_new[h]);
                m[h] = m_new[h];
                l[h] *= alpha;
#pragma unroll
                for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
            }
        }
        if constexpr (BF16) {
            // bf16: weights of two rows rounded to a bf16 pair; V elements of the same dim of the two rows
            // paired with v_perm; one v_dot2_f32_bf16 per (head, dim) covers both rows. The denominator
            // sums the same rounded weights (dot with (1, 1)).
            constexpr uint32_t ONES = 0x3f803f80u;
#pragma unroll
            for (int r = 0; r < R; r += 2) {
                uint32_t pp[G];
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    pp[h] = pack_bf16x2(fast_exp2(s[r][h] - m[h]), fast_exp2(s[r + 1][h] - m[h]));
                    l[h] = dot2_bf16(pp[h], ONES, l[h]);
                }
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t x = pair_lo(t.v[r][v][j], t.v[r + 1][v][j]);
                        const uint32_t y = pair_hi(t.v[r][v][j], t.v[r + 1][v][j]);
#pragma unroll
                        for (int h = 0; h < G; ++h) {
                            acc[h][v * VEC + 2 * j] = dot2_bf16(pp[h], x, acc[h][v * VEC + 2 * j]);
                            acc[h][v * VEC + 2 * j + 1] = dot2_bf16(pp[h], y, acc[h][v * VEC + 2 * j + 1]);
                        }
                    }
            }
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                float vf[EPL];
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int j = 0; j < 4; ++j) vf[v * VEC + j] = __uint_as_float(t.v[r][v][j]);
#pragma unroll
                for (int h = 0; h < G; ++h) {
                    const float p = fast_exp2(s[r][h] - m[h]);
                    l[h] += p;
#pragma unroll
                    for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
                }
            }
        }
    };

    // two-stage pipeline over this wave's tiles: tile, tile + NW, tile + 2 NW, ...
    const int ntiles = (ntok + TILE - 1) / TILE;
    {
        TileRegs<S> ta, tb;
        int tile = wave;
        if (tile < ntiles) issue(tile, ta);
        while (tile < ntiles) {
            const int n1 = tile + NW;
            if (n1 < ntiles) issue(n1, tb);
            compute(tile, ta);
            if (n1 >= ntiles) break;
            const int n2 = n1 + NW;
            if (n2 < ntiles) issue(n2, ta);
            compute(n1, tb);
            tile = n2;
        }
    }

    // merge the RPW groups of the wave (lanes with equal `sub` hold the same elements)
#pragma unroll
    for (int stride = LPT; stride < 64; stride *= 2) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float mo = __shfl_xor(m[h], stride);
            const float lo = __shfl_xor(l[h], stride);
            const float mn = fmaxf(m[h], mo);
            const float a = fast_exp2(m[h] - mn), b = fast_exp2(mo - mn);
            m[h] = mn;
            l[h] = l[h] * a + lo * b;
#pragma unroll
            for (int e = 0; e < EPL; ++e) acc[h][e] = acc[h][e] * a + __shfl_xor(acc[h][e], stride) * b;
        }
    }

    if constexpr (NW > 1) {                           // merge the waves through LDS
        __shared__ float s_m[NW][G];
        __shared__ float s_l[NW][G];
        __shared__ float s_o[NW][G][D];
        if (grp == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                if (sub == 0) {
                    s_m[wave][h] = m[h];
                    s_l[wave][h] = l[h];
                }
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int e = 0; e < VEC; ++e) s_o[wave][h][(v * LPT + sub) * VEC + e] = acc[h][v * VEC + e];
            }
        }
        __syncthreads();
        for (int idx = tid; idx < G * D; idx += 64 * NW) {
            const int h = idx / D, d = idx % D;
            float mm = s_m[0][h];
#pragma unroll
            for (int w = 1; w < NW; ++w) mm = fmaxf(mm, s_m[w][h]);
            float ll = 0.f, oo = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float f = fast_exp2(s_m[w][h] - mm);
                ll += s_l[w][h] * f;
                oo += s_o[w][h][d] * f;
            }
            const int head = kvh * G + h;
            if (!several) {
                const int64_t o = ((int64_t)seq * num_heads + head) * D + d;
                if constexpr (BF16) ((uint16_t *)out)[o] = (uint16_t)f32_to_bf16_rne(oo / ll);
                else ((float *)out)[o] = oo / ll;
            } else {
                const int64_t pidx = ((int64_t)seq * num_heads + head) * max_parts + part;
                ws_o[pidx * D + d] = oo;
                if (d == 0) {
                    ws_m[pidx] = mm;
                    ws_l[pidx] = ll;
                }
            }
        }
    } else {                                          // one wave: group 0 holds the result
        if (grp != 0) return;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const int head = kvh * G + h;
            if (!several) {
                const float inv = 1.0f / l[h];
#pragma unroll
                for (int v = 0; v < NV; ++v) {
                    const int64_t o = ((int64_t)seq * num_heads + head) * D + (v * LPT + sub) * VEC;
                    if constexpr (BF16) {
                        u32x4 pk;
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            pk[j] = f32_to_bf16_rne(acc[h][v * VEC + 2 * j] * inv) |
                                    (f32_to_bf16_rne(acc[h][v * VEC + 2 * j + 1] * inv) << 16);
                        *(u32x4 *)((uint16_t *)out + o) = pk;
                    } else {
                        *(f32x4 *)((float *)out + o) = f32x4{acc[h][v * VEC] * inv, acc[h][v * VEC + 1] * inv,
                                                             acc[h][v * VEC + 2] * inv, acc[h][v * VEC + 3] * inv};
                    }
                }
            } else {
                const int64_t pidx = ((int64_t)seq * num_heads + head) * max_parts + part;
#pragma unroll
                for (int v = 0; v < NV; ++v)
#pragma unroll
                    for (int e = 0; e < VEC; e += 4)
                        *(f32x4 *)&ws_o[pidx * D + (v * LPT + sub) * VEC + e] =
                            f32x4{acc[h][v * VEC + e], acc[h][v * VEC + e + 1], acc[h][v * VEC + e + 2],
                                  acc[h][v * VEC + e + 3]};
                if (sub == 0) {
                    ws_m[pidx] = m[h];
                    ws_l[pidx] = l[h];
                }
            }
        }
    }
}

// Merge the partitions of each (sequence, head): M = max_p m_p, w_p = 2^(m_p - M),
// out = sum_p w_p o_p / sum_p w_p l_p. One workgroup per (kv head, sequence) serves its G heads:
// wave-level reductions give M and the denominator per head, then each thread merges (head, dim)
// outputs with loads coalesced along dim. Sequences that fit one partition were written by the
// decode kernel and exit at once.
constexpr int REDUCE_THREADS = 256;

template <bool BF16, int D, int G>
__global__ void __launch_bounds__(REDUCE_THREADS)
decode_reduce_kernel(void *__restrict__ out, const int32_t *__restrict__ context_lens, int max_context_len,
                     int num_kv_heads, int part_tokens, const float *__restrict__ ws_m, const float *__restrict__ ws_l,
                     const float *__restrict__ ws_o, int max_parts) {
    __shared__ float s_max[G], s_inv[G];
    const int kvh = blockIdx.x, seq = blockIdx.y;
    const int L = min(context_lens[seq], max_context_len);
    const int nparts = (L + part_tokens - 1) / part_tokens;
    if (nparts <= 1) return;
    const int num_heads = num_kv_heads * G;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int h = wave; h < G; h += REDUCE_THREADS / 64) {
        const int64_t pbase = ((int64_t)seq * num_heads + kvh * G + h) * max_parts;
        float mm = M_INIT;
        for (int p = lane; p < nparts; p += 64) mm = fmaxf(mm, ws_m[pbase + p]);
        for (int o = 32; o >= 1; o >>= 1) mm = fmaxf(mm, __shfl_xor(mm, o));
        float ll = 0.f;
        for (int p = lane; p < nparts; p += 64) ll += ws_l[pbase + p] * fast_exp2(ws_m[pbase + p] - mm);
        for (int o = 32; o >= 1; o >>= 1) ll += __shfl_xor(ll, o);
        if (lane == 0) {
            s_max[h] = mm;
            s_inv[h] = 1.0f / ll;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * D; idx += REDUCE_THREADS) {
        const int h = idx / D, d = idx % D;
        const int64_t pbase = ((int64_t)seq * num_heads + kvh * G + h) * max_parts;
        const float mm = s_max[h];
        float oo = 0.f;
        for (int p = 0; p < nparts; ++p) oo += ws_o[(pbase + p) * D + d] * fast_exp2(ws_m[pbase + p] - mm);
        const float res = oo * s_inv[h];
        const int64_t o = ((int64_t)seq * num_heads + kvh * G + h) * D + d;
        if constexpr (BF16) ((uint16_t *)out)[o] = (uint16_t)f32_to_bf16_rne(res);
        else ((float *)out)[o] = res;
    }
}

template <bool BF16, int D, int G, int NV, int R, int NW>
static hipError_t launch_decode_cfg(const DecodeArgs &a, hipStream_t stream) {
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, a.context_lens, a.num_seqs,
                       a.max_context_len, a.part_tokens, a.items, a.ctrl, a.out, a.num_kv_heads * G * D,
                       BF16 ? 2 : 4);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t slots = (int64_t)a.num_seqs * a.num_parts * a.num_kv_heads;
    hipLaunchKernelGGL((decode_kernel<BF16, D, G, NV, R, NW>), dim3((unsigned)slots), dim3(64 * NW), 0, stream, a.out,
                       a.query, (const u32x4 *)a.key_cache, (const u32x4 *)a.value_cache, a.block_tables,
                       a.bt_stride, a.items, a.ctrl, a.num_kv_heads, a.num_blocks, a.log2_bs, a.part_tokens,
                       a.scale_log2e, a.ws_m, a.ws_l, a.ws_o, a.num_parts);
    e = hipGetLastError();
    if (e != hipSuccess || a.num_parts <= 1) return e;
    hipLaunchKernelGGL((decode_reduce_kernel<BF16, D, G>), dim3(a.num_kv_heads, a.num_seqs), dim3(REDUCE_THREADS), 0,
                       stream, a.out, a.context_lens, a.max_context_len, a.num_kv_heads, a.part_tokens, a.ws_m, a.ws_l,
                       a.ws_o, a.num_parts);
    return hipGetLastError();
}

// Kernel shape per (dtype, head_dim, group): vectors per lane NV, tile depth R, waves per workgroup NW.
#ifndef PKV_DECODE_NW
#define PKV_DECODE_NW 1
#endif
#ifndef PKV_DECODE_R2
#define PKV_DECODE_R2 2      // tile depth when a lane holds two vectors of a row
#endif
template <bool BF16, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    constexpr int VPR = D / (BF16 ? 8 : 4);
    constexpr int NV = (VPR / ((G <= 4) ? 2 : 1) > 16) ? VPR / 16 : ((G <= 4) ? 2 : 1);
    constexpr int R = (NV == 1) ? 2 * PKV_DECODE_R2 : (NV == 2 ? PKV_DECODE_R2 : 1);
    return launch_decode_cfg<BF16, D, G, NV, R, PKV_DECODE_NW>(a, stream);
}

template <bool BF16, int D>
static hipError_t launch_decode_d(const DecodeArgs &a, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_decode_t<BF16, D, 1>(a, stream);
        case 2: return launch_decode_t<BF16, D, 2>(a, stream);
        case 3: return launch_decode_t<BF16, D, 3>(a, stream);
        case 4: return launch_decode_t<BF16, D, 4>(a, stream);
        case 5: return launch_decode_t<BF16, D, 5>(a, stream);
        case 6: return launch_decode_t<BF16, D, 6>(a, stream);
        case 7: return launch_decode_t<BF16, D, 7>(a, stream);
        case 8: return launch_decode_t<BF16, D, 8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(const DecodeArgs &a, bool bf16, int head_dim, int group, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (bf16) return head_dim == 128 ? launch_decode_d<true, 128>(a, group, stream)
                                     : launch_decode_d<true, 64>(a, group, stream);
    return head_dim == 128 ? launch_decode_d<false, 128>(a, group, stream)
                           : launch_decode_d<false, 64>(a, group, stream);
}

int decode_max_part_blocks() { return MAX_PART_BLOCKS; }

}  // namespace pkv
