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
// Work decomposition. A part is a run of tokens of one sequence; a unit is a part x one kv head, and
// one wave serves all G query heads of its kv head, so every K/V byte is read once. A one-workgroup
// plan kernel reads context_lens on the device and cuts every sequence into parts whose length is
// chosen from the actual lengths of the batch, so that the batch becomes about as many units of
// equal size as the GPU holds resident waves (long sequences are split, short ones stay whole); it
// lists the parts longest first (a counting sort on the length). One wave processes a unit at a time. A sequence of one part writes its
// output directly; otherwise each part writes an unnormalised partial (running max m, sum l,
// accumulator o, fp32) and the reduce kernel merges them with the log-sum-exp rule.
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
#include <algorithm>
#include <climits>

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

// A run trusts its work list only when the plan's key in the control block equals its own (same sizes, so
// the same workspace layout and unit bounds). The words are wave-uniform scalar loads; on a mismatch the
// kernel raises the error word and returns before any other memory access.
__device__ __forceinline__ bool plan_key_ok(int *ctrl, const PlanKey &key) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) ok &= ctrl[CTRL_KEY + i] == key.w[i];
    if (!ok && threadIdx.x == 0) ctrl[CTRL_ERR] = 1;
    return ok;
}

#ifndef PKV_PLAN_THREADS
#define PKV_PLAN_THREADS 256      // four waves: fewer waves meet at each of the plan's barriers
#endif
constexpr int PLAN_THREADS = PKV_PLAN_THREADS;
constexpr int PLAN_WAVES = PLAN_THREADS / 64;
constexpr int PLAN_BUCKETS = 64;
constexpr int DECODE_TILE = 32;               // part lengths are multiples of this many tokens

// Inclusive prefix (sum, or max) over the 64 lanes of a wave, with DPP moves instead of LDS permutes:
// shifts by 1, 2, 4 and 8 lanes inside each 16-lane row, then lane 15 of rows 0 and 2 combined into rows 1
// and 3, then lane 31 into rows 2 and 3. Lanes a move has no source for take the identity. All 64 lanes
// must be active.
template <bool MAX>
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int id = MAX ? INT_MIN : 0;
    auto op = [](int a, int b) { return MAX ? max(a, b) : a + b; };
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x111, 0xf, 0xf, false));     // row_shr:1
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x112, 0xf, 0xf, false));     // row_shr:2
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x114, 0xf, 0xf, false));     // row_shr:4
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x118, 0xf, 0xf, false));     // row_shr:8
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x142, 0xa, 0xf, false));     // row_bcast:15
    v = op(v, __builtin_amdgcn_update_dpp(id, v, 0x143, 0xc, 0xf, false));     // row_bcast:31
    return v;
}
// the wave's total (sum or max), wave-uniform
__device__ __forceinline__ int wave_total_sum(int v) { return __builtin_amdgcn_readlane(wave_incl_scan<false>(v), 63); }
__device__ __forceinline__ int wave_total_max(int v) { return __builtin_amdgcn_readlane(wave_incl_scan<true>(v), 63); }

// Exclusive prefix sum of v over the plan workgroup; *total gets the sum. Every thread must call it.
__device__ int plan_exclusive_scan(int v, int *s_wave, int *total) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int x = wave_incl_scan<false>(v);
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < PLAN_WAVES; ++w) {
        const int sw = s_wave[w];
        before += w < wave ? sw : 0;
        all += sw;
    }
    __syncthreads();                              // s_wave is reused by the next call
    *total = all;
    return before + x - v;
}

// Work list. Sequence i (L_i tokens, context_lens clamped to [0, max_context_len], t_i = ceil(L_i / 32)
// tiles of 32 tokens) is cut into n_i parts of len_i = 32 ceil(t_i / n_i) tokens, the last part taking the
// rest, with
//   n_i = max(1, round(t_i / g), ceil(t_i / max_tiles))      (then recounted as ceil(t_i / len_i) tiles)
// so parts are about g tiles and no part's block-table slice outgrows a lane register. With cap =
// min_strata W units (W = workers, unit = part x kv head, H = Hkv, T = sum t_i),
//   g = max(min_tiles, ceil(H T / cap)),
// which cuts the batch into about cap units of equal size. When every sequence fits one unit per worker
// (U_min = H sum_i ceil(t_i / max_tiles) <= cap) but rounding leaves U > cap units, g grows (to at least
// ceil(g U / cap)) and the cut is redone until U <= cap: the few units past a stratum would otherwise run
// after all the others, each a whole part long. (U_min is summed only for such a batch, and only when the
// batch has at most cap / H sequences, which any batch that fits has.)
// items[k] = {seq, first token, tokens, partial slot (-1 when the sequence is one part)}, longest first
// (64-bucket counting sort; order inside a bucket is arbitrary and every unit writes its own output, so
// results do not depend on it). seq_info[i] = {first partial slot, n_i, len_i, L_i}; ctrl[0] = number of
// parts (sequences with L_i = 0 have no parts; the reduce kernel writes their zero outputs). red_list gets
// the sequences the reduce kernel has work for (split into parts, or empty; ctrl[CTRL_RED] of them, in any
// order). One workgroup of PLAN_THREADS threads; thread t owns sequences t + k * PLAN_THREADS, and keeps the
// first PLAN_REG of them in registers (larger batches re-read seq_info).
constexpr int PLAN_REG = 4;

__device__ void plan_body(const int32_t *__restrict__ context_lens, int num_seqs, int max_context_len, int num_kv_heads,
                          int workers, int min_strata, int max_tiles, int min_tiles, int4 *__restrict__ items,
                          int4 *__restrict__ seq_info, int *__restrict__ red_list, int *__restrict__ ctrl,
                          const PlanKey &key) {
    __shared__ int s_wave[PLAN_WAVES];
    __shared__ int hist[PLAN_BUCKETS];
    __shared__ int offs[PLAN_BUCKETS];
    __shared__ int s_tiles, s_maxlen, s_umin, s_red;
    const int tid = threadIdx.x;
    if (tid < PLAN_BUCKETS) hist[tid] = 0;
    if (tid == 0) {
        s_tiles = 0;
        s_maxlen = 1;
        s_umin = -1;
        s_red = 0;
    }
    auto clen = [&](int i) { return max(0, min(context_lens[i], max_context_len)); };
    const bool wave_lead = (tid & 63) == 0;
    int lreg[PLAN_REG];
    int t = 0;
#pragma unroll
    for (int k = 0; k < PLAN_REG; ++k) {
        const int i = tid + k * PLAN_THREADS;
        lreg[k] = i < num_seqs ? clen(i) : 0;
        t += (lreg[k] + DECODE_TILE - 1) / DECODE_TILE;
    }
    for (int i = tid + PLAN_REG * PLAN_THREADS; i < num_seqs; i += PLAN_THREADS)
        t += (clen(i) + DECODE_TILE - 1) / DECODE_TILE;
    t = wave_total_sum(t);
    __syncthreads();                                  // s_tiles, s_umin, hist initialised
    if (wave_lead) atomicAdd(&s_tiles, t);
    __syncthreads();
    const int64_t H = num_kv_heads, cap = (int64_t)workers * min_strata;
    const int64_t glo = (H * s_tiles + cap - 1) / cap;
    int target = (int)(glo > min_tiles ? (glo < max_tiles ? glo : max_tiles) : min_tiles);
    // U_min, computed only when a cut overshoots cap and the batch could fit (num_seqs H <= cap)
    auto fits = [&]() {
        if (s_umin < 0) {                             // uniform: s_umin is read after a barrier
            int um = 0;
#pragma unroll
            for (int k = 0; k < PLAN_REG; ++k) um += ((lreg[k] + DECODE_TILE - 1) / DECODE_TILE + max_tiles - 1) / max_tiles;
            for (int i = tid + PLAN_REG * PLAN_THREADS; i < num_seqs; i += PLAN_THREADS)
                um += ((clen(i) + DECODE_TILE - 1) / DECODE_TILE + max_tiles - 1) / max_tiles;
            um = wave_total_sum(um);
            __syncthreads();
            if (tid == 0) s_umin = 0;
            __syncthreads();
            if (wave_lead) atomicAdd(&s_umin, um);
            __syncthreads();
        }
        return H * s_umin <= cap;
    };

    // parts per sequence and their partial slots (exclusive scan, PLAN_THREADS sequences at a time)
    int4 sreg[PLAN_REG];
    int carry, my_max;
    for (;;) {                                        // uniform over the workgroup
        carry = 0;
        my_max = 1;
        for (int k = 0, base = 0; base < num_seqs; ++k, base += PLAN_THREADS) {
            const int i = base + tid;
            int L = 0, n = 0, len = 0;
            if (i < num_seqs) {
                if (k < PLAN_REG) {
                    L = lreg[0];
#pragma unroll
                    for (int r = 1; r < PLAN_REG; ++r)
                        if (r == k) L = lreg[r];
                } else {
                    L = clen(i);
                }
                const int tiles = (L + DECODE_TILE - 1) / DECODE_TILE;
                if (tiles > 0) {
                    n = max(max(1, (tiles + target / 2) / target), (tiles + max_tiles - 1) / max_tiles);
                    const int lt = (tiles + n - 1) / n;
                    n = (tiles + lt - 1) / lt;
                    len = lt * DECODE_TILE;
                }
            }
            int chunk;
            const int first = carry + plan_exclusive_scan(n, s_wave, &chunk);
            const int4 si = make_int4(first, n, len, L);
#pragma unroll
            for (int r = 0; r < PLAN_REG; ++r)
                if (r == k) sreg[r] = si;
            if (i < num_seqs) {
                seq_info[i] = si;
                if (n > 0) my_max = max(my_max, min(len, L));
            }
            carry += chunk;
        }
        if (H * carry <= cap || target >= max_tiles || (int64_t)num_seqs * H > cap || !fits()) break;
        const int64_t grown = ((int64_t)target * H * carry + cap - 1) / cap;
        target = (int)(grown > target + 1 ? (grown < max_tiles ? grown : max_tiles) : target + 1);
    }
    if (tid == 0) {
        ctrl[CTRL_PARTS] = carry;
#pragma unroll
        for (int w = 0; w < 8; ++w) ctrl[CTRL_KEY + w] = key.w[w];
        ctrl[CTRL_ERR] = 0;
    }
    my_max = wave_total_max(my_max);
    if (wave_lead) atomicMax(&s_maxlen, my_max);
    __syncthreads();
    const int maxlen = s_maxlen;
    auto bucket = [&](int ntok) {
        return min(PLAN_BUCKETS - 1, (int)((int64_t)(maxlen - ntok) * PLAN_BUCKETS / maxlen));
    };
    auto count = [&](const int4 &si) {
        if (si.y <= 0) return;
        if (si.y > 1) atomicAdd(&hist[bucket(si.z)], si.y - 1);
        atomicAdd(&hist[bucket(si.w - (si.y - 1) * si.z)], 1);
    };
#pragma unroll
    for (int k = 0; k < PLAN_REG; ++k)
        if (tid + k * PLAN_THREADS < num_seqs) count(sreg[k]);
    for (int i = tid + PLAN_REG * PLAN_THREADS; i < num_seqs; i += PLAN_THREADS) count(seq_info[i]);
    __syncthreads();
    if (tid < 64) {                                   // exclusive scan of the 64 buckets in one wave
        const int h = hist[tid];
        offs[tid] = wave_incl_scan<false>(h) - h;
    }
    __syncthreads();
    auto emit = [&](int i, const int4 &si) {      // n - 1 full parts share a bucket: one reservation
        if (si.y != 1) red_list[atomicAdd(&s_red, 1)] = i;    // split or empty: the reduce kernel's work
        if (si.y <= 0) return;
        const int pfull = si.y > 1 ? atomicAdd(&offs[bucket(si.z)], si.y - 1) : 0;
        for (int p = 0; p + 1 < si.y; ++p) items[pfull + p] = make_int4(i, p * si.z, si.z, si.x + p);
        const int start = (si.y - 1) * si.z;
        items[atomicAdd(&offs[bucket(si.w - start)], 1)] = make_int4(i, start, si.w - start, si.y > 1 ? si.x + si.y - 1 : -1);
    };
#pragma unroll
    for (int k = 0; k < PLAN_REG; ++k)
        if (tid + k * PLAN_THREADS < num_seqs) emit(tid + k * PLAN_THREADS, sreg[k]);
    for (int i = tid + PLAN_REG * PLAN_THREADS; i < num_seqs; i += PLAN_THREADS) emit(i, seq_info[i]);
    __syncthreads();
    if (tid == 0) ctrl[CTRL_RED] = s_red;
}

__global__ void __launch_bounds__(PLAN_THREADS)
decode_plan_kernel(const int32_t *__restrict__ context_lens, int num_seqs, int max_context_len, int num_kv_heads,
                   int workers, int min_strata, int max_tiles, int min_tiles, int4 *__restrict__ items,
                   int4 *__restrict__ seq_info, int *__restrict__ red_list, int *__restrict__ ctrl, PlanKey key) {
    plan_body(context_lens, num_seqs, max_context_len, num_kv_heads, workers, min_strata, max_tiles, min_tiles, items,
              seq_info, red_list, ctrl, key);
}

// A decode step's store and plan in one launch: workgroup 0 builds the plan (it reads only context_lens),
// the others move the new rows into their slots (the store kernel's work, PLAN_THREADS pieces each). The two
// touch disjoint memory, and the decode kernel that reads both follows in stream order.
template <int CHUNKS>
__global__ void __launch_bounds__(PLAN_THREADS)
store_and_plan_kernel(const u32x4 *__restrict__ key, const u32x4 *__restrict__ value, u32x4 *__restrict__ key_cache,
                      u32x4 *__restrict__ value_cache, const int32_t *__restrict__ slot_mapping, int64_t num_rows,
                      int block_size, int num_blocks,
                      const int32_t *__restrict__ context_lens, int num_seqs, int max_context_len, int num_kv_heads,
                      int workers, int min_strata, int max_tiles, int min_tiles, int4 *__restrict__ items,
                      int4 *__restrict__ seq_info, int *__restrict__ red_list, int *__restrict__ ctrl, PlanKey pkey) {
    if (blockIdx.x == 0) {
        plan_body(context_lens, num_seqs, max_context_len, num_kv_heads, workers, min_strata, max_tiles, min_tiles,
                  items, seq_info, red_list, ctrl, pkey);
        return;
    }
    store_piece<CHUNKS>((int64_t)(blockIdx.x - 1) * PLAN_THREADS + threadIdx.x, key, value, key_cache, value_cache,
                        slot_mapping, num_rows, num_kv_heads, block_size, num_blocks);
}

template <bool BF16, int D, int G, int NV_, int R_, int NW_>
__global__ void __launch_bounds__(64 * NW_)
decode_kernel(void *__restrict__ out, const void *__restrict__ query, const u32x4 *__restrict__ key_cache,
              const u32x4 *__restrict__ value_cache, const int32_t *__restrict__ block_tables, int bt_stride,
              const int4 *__restrict__ items, int *__restrict__ ctrl, PlanKey key, int num_kv_heads,
              int64_t num_blocks, int log2_bs, float scale_log2e,
              float *__restrict__ ws_m, float *__restrict__ ws_l, float *__restrict__ ws_o) {
    using S = DecodeShape<BF16, D, G, NV_, R_, NW_>;
    if (!plan_key_ok(ctrl, key)) return;
    constexpr int NV = S::NV, LPT = S::LPT, RPW = S::RPW, R = S::R, TILE = S::TILE, EPL = S::EPL, VEC = S::VEC;
    constexpr int NW = S::NW;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int grp = lane / LPT, sub = lane % LPT;
    const int num_heads = num_kv_heads * G;

    // unit in longest-first order; workgroups past the list exit
    const int unit = blockIdx.x;
    if (unit >= ctrl[CTRL_PARTS] * num_kv_heads) return;
    const int4 item = items[unit / num_kv_heads];
    const int kvh = unit % num_kv_heads;
    const int seq = item.x, start = item.y, ntok = item.z, pslot = item.w;
    const bool several = pslot >= 0;

    // the part's block-table slice (<= 64 ids), one id per lane
    const int first_blk = start >> log2_bs;
    const int nbp = ((start + ntok - 1) >> log2_bs) - first_blk + 1;
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
                const int64_t pidx = (int64_t)pslot * num_heads + head;
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
                const int64_t pidx = (int64_t)pslot * num_heads + head;
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

// Buffer descriptor word 3 for raw (untyped, unswizzled) buffers on gfx9-family GPUs.
constexpr int BUF_RSRC_W3 = 0x00020000;

// 16- and 8-byte loads through a buffer descriptor; non-temporal unless PKV_DECODE_NT is 0.
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, PKV_DECODE_NT ? 2 : 0);
}
__device__ __forceinline__ u32x2 buffer_load8(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, PKV_DECODE_NT ? 2 : 0);
}
__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, int byte_off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, byte_off, 0, PKV_DECODE_NT ? 2 : 0);
}

// Four-bit codes u (element e of a 32-bit word in bits 4 e .. 4 e + 3) to bf16 pairs without conversion
// instructions: 0x4300 | u is the bf16 of 128 + u (the exponent of 128 puts the mantissa's last bit at 1),
// so pair k = ((w >> 4 k) & 0x000f000f) | 0x43004300 holds elements k and k + 4 as 128 + u. With u = q + 8
// the values are 136 + q; the decode subtracts 136 times the matching sums (I4_BIAS).
constexpr float I4_BIAS = 136.0f;
// The mask (in a scalar register) and the exponent bits (in a vector register) are held in registers the
// compiler cannot see through, so each pair is one v_and_or_b32 (after a shift for K > 0): these encodings
// take neither a literal nor two scalar operands.
struct NibbleConsts {
    uint32_t mask, bits;
};
__device__ __forceinline__ NibbleConsts nibble_consts() {
    NibbleConsts c;
    asm("s_mov_b32 %0, 0x000f000f" : "=s"(c.mask));
    asm("v_mov_b32 %0, 0x43004300" : "=v"(c.bits));
    return c;
}
template <int K>
__device__ __forceinline__ uint32_t nibble_pair_to_bf16x2(uint32_t w, const NibbleConsts &c) {
    return ((w >> (4 * K)) & c.mask) | c.bits;
}

// Registers of one 32-token tile of the matrix-core decode: bf16 rows, or 8-bit codes plus per-row scales,
// or 4-bit codes plus per-row scales.
template <bool Q8, bool I4 = false>
struct MfmaTile {
    u32x4 k[2][4];
    u32x4 v[2][4];
    bool live[2];                           // group's block id lies in the pool
};
template <>
struct MfmaTile<true, false> {
    u32x4 k[2][2];                          // per group: dims 16 b .. +16 and 64 + 16 b .. +16 of row n
    u32x2 v[2][4];                          // per group and i: dims 8 n .. +8 of row 4 b + i
    f32x4 ks[2], vs[2];                     // scales of rows 4 b .. 4 b + 3 of each group
    bool live[2];
};
template <>
struct MfmaTile<true, true> {
    u32x4 k[2];                             // per group: dims 32 b .. 32 b + 32 of row n (word c: 32 b + 8 c ..)
    uint32_t v[2][4];                       // per group and i: dims 8 n .. +8 of row 4 b + i
    f32x4 ks[2], vs[2];
    bool live[2];
};

// The same units on the matrix cores (bf16, head_dim 128, block_size >= 16), with a persistent grid of
// one workgroup per compute unit whose waves take units from the list until it is done (see the kernel).
// The G query heads of the kv head are the N = 16 columns of v_mfma_f32_16x16x32_bf16 (columns past
// G carry zero queries and are never written), so a 32-token tile costs 8 MFMAs per product and the
// vector ALU keeps only the softmax.
// A tile is two 16-token groups g. Lane l = n + 16 b (n = l % 16, b = l / 16) holds:
//   K (A operand of S^T = K Q^T): token 16 g + n, dims 32 c + 8 b .. +8 for c = 0..3 (each load covers
//     64 contiguous bytes of 16 rows);
//   Q (B operand): head n, the same dims (zero for n >= G);
//   S^T (output): head n, tokens 16 g + 4 b + i, i = 0..3;
//   V: tokens 16 g + 4 b + i, dims 8 n .. 8 n + 8 (each load covers 4 whole rows);
//   P^T (B operand of O^T = V^T P^T): the rounded weights of the lane's own S^T values, reduction
//     element e = 4 g + i <-> token 16 g + 4 b + i;
//   V^T (A operand, one MFMA per j = 0..7): row n <-> dim 8 n + j, element e = element j of the lane's V
//     row of token (g, i), paired with v_perm: the data never leaves the lane;
//   O^T (output of MFMA j): head n, dims 8 (4 b + i) + j, so the lane ends with dims 32 b .. 32 b + 32.
// The running max of a head is shared by its 4 lanes (max over lane ^ 16, lane ^ 32); the running sum
// is kept per lane and summed when the unit ends.
// The K/V pipeline runs across unit boundaries: while the last tile of a unit is computed, the first
// tile of the wave's next unit is already loading (its work item and block-table slice were fetched
// during the current unit), so a wave pays the dependent-load chain of a unit start only once.
// Block size >= 16 puts each 16-token group in one block: the block id and block base are wave-uniform
// and lanes add 32-bit row offsets.
//
// 8-bit caches (Q8): rows hold one-byte codes with one fp32 scale per (token, kv head): int8 integers, or
// OCP float8 E4M3 values (F8). K codes of a lane are two 16-byte loads (dims 16 b .. +16 and 64 + 16 b .. +16,
// the MFMA reduction order permuted to match, Q loaded in the same order), V codes one 8-byte load per
// token; codes become exact bf16 values in registers (int8: a signed-byte conversion per code; E4M3:
// v_cvt_scalef32_pk_bf16_fp8 with scale 1, two codes per instruction), the K scale multiplies each score,
// and the V scale multiplies each weight before it is rounded to bf16 (the denominator sums the unscaled
// weights).
template <bool F8, int K>
__device__ __forceinline__ uint32_t code_pair_to_bf16x2(uint32_t w) {
    if constexpr (F8) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, K != 0));
    else return i8pair_to_bf16x2(w, K);
}

// Waves of one matrix-core decode workgroup (one workgroup per compute unit): one per SIMD over bf16
// caches; two per SIMD over 8-bit caches, whose tiles carry half the bytes, so a wave alone keeps too
// few of them in flight.
constexpr int DECODE_CU_WAVES_BF16 = 4;
constexpr int DECODE_CU_WAVES_Q8 = 8;
#ifndef PKV_DECODE_CLAIM_LEAD
#define PKV_DECODE_CLAIM_LEAD 3
#endif
constexpr int DECODE_CLAIM_LEAD = PKV_DECODE_CLAIM_LEAD;  // tiles left in a unit when the next is claimed

template <int G, bool Q8, bool F8, bool I4 = false, int NWV = Q8 ? DECODE_CU_WAVES_Q8 : DECODE_CU_WAVES_BF16>
__global__ void __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(2, 2)))
decode_mfma_kernel(void *__restrict__ out, const void *__restrict__ query, const char *__restrict__ key_cache,
                   const char *__restrict__ value_cache, const int32_t *__restrict__ block_tables, int bt_stride,
                   const int4 *__restrict__ items, int *__restrict__ ctrl, PlanKey key, int num_kv_heads,
                   int64_t num_blocks, int log2_bs, float scale_log2e,
                   float *__restrict__ ws_m, float *__restrict__ ws_l, float *__restrict__ ws_o,
                   const float *__restrict__ key_scale, const float *__restrict__ value_scale) {
    static_assert(G >= 1 && G <= 16, "query heads per kv head");
    if (!plan_key_ok(ctrl, key)) return;
    constexpr int D = 128, CH = D / 8;        // 16-byte chunks of a bf16 row
    static_assert(!I4 || (Q8 && !F8), "4-bit codes use the quantized-cache path");
    constexpr int RB = I4 ? D / 2 : Q8 ? D : 2 * D;     // bytes per cache row
    constexpr int TILE = 32;
    constexpr uint32_t ONES = 0x3f803f80u;    // bf16 pair (1, 1)
    const int lane = threadIdx.x & 63, n = lane & 15, b = lane >> 4;
    const int num_heads = num_kv_heads * G;
    const int bs_mask = (1 << log2_bs) - 1;
    const int nunits = ctrl[CTRL_PARTS] * num_kv_heads;
    // Units are dealt to the C workgroups (one per compute unit) from the longest-first list in strata
    // of C: in stratum k workgroup c takes unit k C + c for even k and k C + C - 1 - c for odd k (snake
    // order, so the long units of one stratum pair with the short ones of the next), except that a
    // partial last stratum (k >= 1) runs the other way. Inside the workgroup the waves share its strata
    // through an LDS counter: wave v starts with stratum v and claims each later one shortly before it
    // needs it, so waves that run faster take more of the list and every wave of the compute unit runs
    // until the list is done. (Waves do not run at equal rates: of two waves sharing a SIMD the older
    // one wins arbitration and streams up to twice as fast.) A wave stops at its first stratum whose
    // unit lies past the list.
    // (readfirstlane: without it the compiler treats the grid size and workgroup id as per-lane values, so
    // every unit field derived from them sat in vector registers and each buffer descriptor built from one
    // went through a waterfall loop)
    const int C = __builtin_amdgcn_readfirstlane((int)gridDim.x), cu = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
    auto unit_index = [&](int k) {
        const bool rev = ((k & 1) != 0) != (k > 0 && (k + 1) * C > nunits);
        return k * C + (rev ? C - 1 - cu : cu);
    };
    __shared__ int s_next_stratum;
    if (threadIdx.x == 0) s_next_stratum = NWV;
    __syncthreads();
    auto claim = [&]() {
        int k = 0;
        if (lane == 0) k = atomicAdd(&s_next_stratum, 1);
        return __builtin_amdgcn_readfirstlane(k);
    };
    const int wave_id = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));   // wave-uniform
    const int first = unit_index(wave_id);
    if (first >= nunits) return;

    struct Unit {
        int seq, start, ntok, pslot, kvh, first_blk, ntiles;
    };
    auto load_unit = [&](int uu) {
        const int4 it = items[uu / num_kv_heads];
        Unit x;
        x.seq = it.x;
        x.start = it.y;
        x.ntok = it.z;
        x.pslot = it.w;
        x.kvh = uu % num_kv_heads;
        x.first_blk = it.y >> log2_bs;
        x.ntiles = (it.z + TILE - 1) / TILE;
        return x;
    };
    // the unit's block-table slice (<= 64 ids), one id per lane
    auto load_slice = [&](const Unit &x) {
        const int span = ((x.start + x.ntok - 1) >> log2_bs) - x.first_blk + 1;
        int v = -1;
        if (lane < span && x.first_blk + lane < bt_stride) v = block_tables[(int64_t)x.seq * bt_stride + x.first_blk + lane];
        return v;
    };
    u32x4 qt[4], qn[4];                         // queries of the current unit; of the next one (prefetched)
    auto load_q = [&](const Unit &x, u32x4 (&dst)[4]) {
        const u32x4 *qv = (const u32x4 *)query;
        const int64_t row = ((int64_t)x.seq * num_heads + x.kvh * G + (n < G ? n : 0)) * CH;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int chunk = I4 ? 4 * b + c : Q8 ? (c < 2 ? 2 * b + c : 8 + 2 * b + (c - 2)) : 4 * c + b;
            dst[c] = n < G ? qv[row + chunk] : u32x4{0, 0, 0, 0};
        }
    };

    using Tile = MfmaTile<Q8, I4>;
    // Rows past the unit's end are clamped to its last token (same block: a group past the end is
    // clamped whole), so every lane reads a row holding finite data; such tokens get zero weight.
    // Loads go through buffer descriptors of the group's (block, kv head) slab: wave-uniform base,
    // 32-bit lane offsets, and the hardware range check bounds every access to the slab.
    const uint32_t slab_bytes = (uint32_t)RB << log2_bs;
    auto issue = [&](const Unit &x, int xblk, int tile, Tile &t) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            const int tl0 = tile * TILE + 16 * g;
            const int tlc = min(tl0, x.ntok - 1);
            const int tokc = x.start + tlc;
            const int64_t blk = __builtin_amdgcn_readlane(xblk, (tokc >> log2_bs) - x.first_blk);
            t.live[g] = blk >= 0 && blk < num_blocks;
            // a block outside the pool gets empty descriptors: its loads return zeros (finite K, V and scales)
            const int64_t slab = t.live[g] ? ((blk * num_kv_heads + x.kvh) << log2_bs) : 0;   // first row
            const int range = t.live[g] ? (int)slab_bytes : 0;
            const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(key_cache + slab * RB), (short)0, range, BUF_RSRC_W3);
            const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(value_cache + slab * RB), (short)0, range, BUF_RSRC_W3);
            const int last = x.ntok - 1 - tl0;              // rows past it are clamped to it
            const int r0 = (tokc & bs_mask) - tlc + tl0;    // slab row of token tl0
            if constexpr (I4) {
                t.k[g] = buffer_load16(kr, (r0 + min(n, last)) * RB + 16 * b);
#pragma unroll
                for (int i = 0; i < 4; ++i) t.v[g][i] = buffer_load4(vr, (r0 + min(4 * b + i, last)) * RB + 4 * n);
            } else if constexpr (Q8) {
                const int koff = (r0 + min(n, last)) * RB + 16 * b;
                t.k[g][0] = buffer_load16(kr, koff);
                t.k[g][1] = buffer_load16(kr, koff + 64);
#pragma unroll
                for (int i = 0; i < 4; ++i) t.v[g][i] = buffer_load8(vr, (r0 + min(4 * b + i, last)) * RB + 8 * n);
            }
            if constexpr (Q8) {
                // scales of the 16-row group holding the clamped token (its own rows when the group is live)
                const int srow = (tokc & bs_mask) & ~15;
                const __amdgpu_buffer_rsrc_t ksr = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(key_scale + slab), (short)0, t.live[g] ? 4 << log2_bs : 0, BUF_RSRC_W3);
                const __amdgpu_buffer_rsrc_t vsr = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(value_scale + slab), (short)0, t.live[g] ? 4 << log2_bs : 0, BUF_RSRC_W3);
                t.ks[g] = __builtin_bit_cast(f32x4, buffer_load16(ksr, (srow + 4 * b) * 4));
                t.vs[g] = __builtin_bit_cast(f32x4, buffer_load16(vsr, (srow + 4 * b) * 4));
            } else {
                const int koff = (r0 + min(n, last)) * RB + 16 * b;
#pragma unroll
                for (int c = 0; c < 4; ++c) t.k[g][c] = buffer_load16(kr, koff + 64 * c);
#pragma unroll
                for (int i = 0; i < 4; ++i) t.v[g][i] = buffer_load16(vr, (r0 + min(4 * b + i, last)) * RB + 16 * n);
            }
        }
    };

    const NibbleConsts nc = I4 ? nibble_consts() : NibbleConsts{0u, 0u};
    float m = M_INIT, l = 0.f;
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // 4-bit codes enter the products as 136 + q (nibble_pair_to_bf16x2). Scores then carry 136 times the
    // head's query sum (kcorr, subtracted from every score), and the accumulators 136 times the sum of the
    // bf16 weights they took (vsum, kept beside l and subtracted in finish). The K operand pairs elements
    // k and k + 4 of each 8-element chunk, so the query chunk is reordered to match when the unit starts.
    float kcorr = 0.f, vsum = 0.f;
    auto prep_q = [&]() {
        float qs = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 w = qt[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) qs = dot2_bf16(w[e], ONES, qs);
            qt[c] = u32x4{pair_lo(w[0], w[2]), pair_hi(w[0], w[2]), pair_lo(w[1], w[3]), pair_hi(w[1], w[3])};
        }
        kcorr = I4_BIAS * lane_blocks_sum(qs);
    };

    auto compute = [&](const Unit &x, int tile, Tile &t) {
        // masked tokens: past the unit's end (only in its last tile; their rows repeat the unit's last token),
        // or in a block outside the pool (its loads returned zeros, see issue). Group g holds tile tokens
        // 16 g .. 16 g + 15, of which the first lim[g] (wave-uniform) are real; a lane's token 4 b + i of the
        // group is kept iff 4 b + i < lim[g] (one compare, no branch).
        int lim[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) lim[g] = t.live[g] ? x.ntok - (tile * TILE + 16 * g) : 0;
        // bf16 operands of the tile (int8 codes are converted exactly)
        u32x4 tk[2][4], tv[2][4];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            if constexpr (I4) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t w = t.k[g][c];
                    tk[g][c] = u32x4{nibble_pair_to_bf16x2<0>(w, nc), nibble_pair_to_bf16x2<1>(w, nc),
                                     nibble_pair_to_bf16x2<2>(w, nc), nibble_pair_to_bf16x2<3>(w, nc)};
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t w = t.v[g][i];
                    tv[g][i] = u32x4{nibble_pair_to_bf16x2<0>(w, nc), nibble_pair_to_bf16x2<1>(w, nc),
                                     nibble_pair_to_bf16x2<2>(w, nc), nibble_pair_to_bf16x2<3>(w, nc)};
                }
            } else if constexpr (Q8) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 w = t.k[g][c >> 1];
                    const uint32_t w0 = (c & 1) ? w[2] : w[0], w1 = (c & 1) ? w[3] : w[1];
                    tk[g][c] = u32x4{code_pair_to_bf16x2<F8, 0>(w0), code_pair_to_bf16x2<F8, 1>(w0),
                                     code_pair_to_bf16x2<F8, 0>(w1), code_pair_to_bf16x2<F8, 1>(w1)};
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tv[g][i] = u32x4{code_pair_to_bf16x2<F8, 0>(t.v[g][i][0]), code_pair_to_bf16x2<F8, 1>(t.v[g][i][0]),
                                     code_pair_to_bf16x2<F8, 0>(t.v[g][i][1]), code_pair_to_bf16x2<F8, 1>(t.v[g][i][1])};
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) tk[g][c] = t.k[g][c];
#pragma unroll
                for (int i = 0; i < 4; ++i) tv[g][i] = t.v[g][i];
            }
        }
        f32x4 s[2];
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            s[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) s[g] = mfma16x16x32(tk[g][c], qt[c], s[g]);
        }
        float xs[2][4], vsc[2][4];
        float mx = -INFINITY;
#pragma unroll
        for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = 4 * b + i < lim[g];
                float sc = scale_log2e;
                vsc[g][i] = 1.f;
                if constexpr (Q8) {
                    sc *= t.ks[g][i];
                    vsc[g][i] = ok ? t.vs[g][i] : 0.f;
                }
                xs[g][i] = ok ? (I4 ? s[g][i] - kcorr : s[g][i]) * sc : -INFINITY;
                mx = fmaxf(mx, xs[g][i]);
            }
        mx = lane_blocks_max(mx);
        const float m_new = fmaxf(m, mx);
        if (__builtin_amdgcn_ballot_w64(m_new > m)) {   // rescale only when a running max grew
            const float alpha = fast_exp2(m - m_new);
            m = m_new;
            l *= alpha;
            if constexpr (I4) vsum *= alpha;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[j] *= alpha;
        }
        u32x4 pb;
        if constexpr (Q8) {
#pragma unroll
            for (int g = 0; g < 2; ++g)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const float p0 = fast_exp2(xs[g][2 * h2] - m), p1 = fast_exp2(xs[g][2 * h2 + 1] - m);
                    l += p0 + p1;
                    pb[2 * g + h2] = pack_bf16x2(p0 * vsc[g][2 * h2], p1 * vsc[g][2 * h2 + 1]);
                }
            if constexpr (I4) {
#pragma unroll
                for (int w = 0; w < 4; ++w) vsum = dot2_bf16(pb[w], ONES, vsum);
            }
        } else {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                pb[2 * g] = pack_bf16x2(fast_exp2(xs[g][0] - m), fast_exp2(xs[g][1] - m));
                pb[2 * g + 1] = pack_bf16x2(fast_exp2(xs[g][2] - m), fast_exp2(xs[g][3] - m));
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) l = dot2_bf16(pb[w], ONES, l);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int w = j >> 1;
            u32x4 a;
            if (j & 1) {
                a[0] = pair_hi(tv[0][0][w], tv[0][1][w]);
                a[1] = pair_hi(tv[0][2][w], tv[0][3][w]);
                a[2] = pair_hi(tv[1][0][w], tv[1][1][w]);
                a[3] = pair_hi(tv[1][2][w], tv[1][3][w]);
            } else {
                a[0] = pair_lo(tv[0][0][w], tv[0][1][w]);
                a[1] = pair_lo(tv[0][2][w], tv[0][3][w]);
                a[2] = pair_lo(tv[1][0][w], tv[1][1][w]);
                a[3] = pair_lo(tv[1][2][w], tv[1][3][w]);
            }
            acc[j] = mfma16x16x32(a, pb, acc[j]);
        }
    };

    // write the unit's result (final output, or its partial slot) and reset the softmax state
    auto finish = [&](const Unit &x) {
        const float lt = lane_blocks_sum(l);
        float corr = 0.f;                       // 4-bit codes: 136 times the weights' sum (see prep_q)
        if constexpr (I4) {
            corr = I4_BIAS * lane_blocks_sum(vsum);
        }
        // accumulator of dim offset e (0..7) of the lane's 8-dim run i: MFMA j = e for bf16 and 8-bit
        // codes; for 4-bit codes MFMA j holds offset j / 2 + 4 (j % 2), so e comes from j = 2 e (e < 4) or
        // 2 (e - 4) + 1
        auto od = [&](int e, int i) {
            if constexpr (I4) return acc[e < 4 ? 2 * e : 2 * (e - 4) + 1][i] - corr;
            else return acc[e][i];
        };
        if (n < G) {
            const int head = x.kvh * G + n;
            if (x.pslot < 0) {
                const float inv = 1.0f / lt;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    u32x4 pk;
#pragma unroll
                    for (int w = 0; w < 4; ++w) pk[w] = pack_bf16x2(od(2 * w, i) * inv, od(2 * w + 1, i) * inv);
                    *(u32x4 *)((uint16_t *)out + ((int64_t)x.seq * num_heads + head) * D + 32 * b + 8 * i) = pk;
                }
            } else {
                const int64_t pidx = (int64_t)x.pslot * num_heads + head;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float *o = ws_o + pidx * D + 32 * b + 8 * i;
                    *(f32x4 *)o = f32x4{od(0, i), od(1, i), od(2, i), od(3, i)};
                    *(f32x4 *)(o + 4) = f32x4{od(4, i), od(5, i), od(6, i), od(7, i)};
                }
                if (b == 0) {
                    ws_m[pidx] = m;
                    ws_l[pidx] = lt;
                }
            }
        }
        m = M_INIT;
        l = 0.f;
        vsum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    };

    Unit cur = load_unit(first);
    int cur_blk = load_slice(cur);
    load_q(cur, qt);
    // The next unit is claimed when the current one has DECODE_CLAIM_LEAD tiles left (at once for shorter
    // units): late enough that waves which run faster claim more of the workgroup's list, early enough
    // that its work item, then its block-table slice and queries, then its first tile arrive behind the
    // current unit's last tiles.
    Unit nxt = cur;
    bool claimed = false, has_next = false, nxt_ready = false;
    int nxt_blk = -1, claim_ct = 0;
    int ct = 0;                                 // tile of `cur` being computed
    auto claim_next = [&]() {
        const int nu = unit_index(claim());
        has_next = nu < nunits;
        if (has_next) nxt = load_unit(nu);
        claimed = true;
        claim_ct = ct;
    };
    auto prepare_next = [&]() {                 // block-table slice and queries of the claimed unit
        nxt_blk = load_slice(nxt);
        load_q(nxt, qn);
        nxt_ready = true;
    };
    if (cur.ntiles <= DECODE_CLAIM_LEAD) claim_next();

    // one pipeline step: load the tile after `ct` into B (the next unit's first tile when `ct` is the
    // last), compute tile `ct` from A, then advance; false once the wave's last unit is written
    // (one issue site: after the wave's last tile it reloads that tile, which nothing reads)
    auto step = [&](Tile &A, Tile &B) -> bool {
        const bool last = ct + 1 >= cur.ntiles;
        if (last && !claimed) claim_next();
        const bool go_next = last && has_next;
        if (go_next && !nxt_ready) prepare_next();
        issue(go_next ? nxt : cur, go_next ? nxt_blk : cur_blk, go_next ? 0 : (last ? ct : ct + 1), B);
        compute(cur, ct, A);
        if (!last) {
            ++ct;
        } else {
            finish(cur);
            if (!has_next) return false;
            cur = nxt;
            cur_blk = nxt_blk;
            ct = 0;
#pragma unroll
            for (int c = 0; c < 4; ++c) qt[c] = qn[c];
            if constexpr (I4) prep_q();         // here, not in compute: a per-tile test there became selects
            claimed = false;
            nxt_ready = false;
        }
        if (!claimed) {
            if (cur.ntiles - ct <= DECODE_CLAIM_LEAD) claim_next();
        } else if (has_next && !nxt_ready && ct > claim_ct) {
            prepare_next();                     // the claimed unit's item has had a step to arrive
        }
        return true;
    };

    Tile ta, tb;
    issue(cur, cur_blk, 0, ta);
    if constexpr (I4) prep_q();
    while (step(ta, tb) && step(tb, ta)) {
    }
}

// Merge the parts of each (sequence, head): M = max_p m_p, w_p = 2^(m_p - M),
// out = sum_p w_p o_p / sum_p w_p l_p. The plan lists the sequences with work here (split into parts, or
// empty: those get zeros); workgroup (x, y) serves heads x * hpb .. + hpb of list entries y, y + Y, ...
// (hpb in {1, 2, 4, 8}). Its threads are hpb heads x PL = 8 / hpb part lanes x D/4 dim groups: a thread merges
// dims 4 dg .. +4 of the parts p = pl mod PL with 16-byte loads (running max, so each part's m, l, o load in
// one round trip), and the part lanes are merged through LDS by the same rule. Sequences of one part were
// written by the decode kernel; when none is split or empty the list is empty and every workgroup exits
// after one load.
constexpr int REDUCE_THREADS = 256;
constexpr int REDUCE_WGS = 1024;             // workgroups the reduce grid aims at

template <bool BF16, int D>
__global__ void __launch_bounds__(REDUCE_THREADS)
decode_reduce_kernel(void *__restrict__ out, const int4 *__restrict__ seq_info, const int *__restrict__ red_list,
                     int num_heads, int hpb, const float *__restrict__ ws_m, const float *__restrict__ ws_l,
                     const float *__restrict__ ws_o, int *__restrict__ ctrl, PlanKey key) {
    constexpr int DG = D / 4, SLOTS = REDUCE_THREADS / DG;          // SLOTS = head slots x part lanes
    __shared__ f32x4 s_o[SLOTS][DG];
    __shared__ float s_l[SLOTS], s_m[SLOTS];
    if (!plan_key_ok(ctrl, key)) return;
    const int count = ctrl[CTRL_RED];
    const int PL = SLOTS / hpb;
    const int t = threadIdx.x, slot = t / DG, dg = t % DG;
    const int hs = slot / PL, pl = slot % PL;
    const int head = blockIdx.x * hpb + hs;
    const bool active = head < num_heads;
    for (int e = blockIdx.y; e < count; e += gridDim.y) {           // uniform over the workgroup
        const int seq = red_list[e];
        const int4 si = seq_info[seq];
        const int nparts = si.y;
        if (nparts == 0) {                       // empty context: zero outputs for this workgroup's heads
            const int h0 = blockIdx.x * hpb, nh = min(hpb, num_heads - h0);
            const int64_t base = ((int64_t)seq * num_heads + h0) * D;
            for (int x = t; x < nh * D; x += REDUCE_THREADS) {
                if constexpr (BF16) ((uint16_t *)out)[base + x] = 0;
                else ((float *)out)[base + x] = 0.f;
            }
            continue;
        }
        float ll = 0.f;
        f32x4 oo = {0.f, 0.f, 0.f, 0.f};
        // one pass per part lane with a running max (each part's m, l and o load together), then the part
        // lanes are merged with the same rule through LDS
        float mm = M_INIT;
        if (active) {
            const int64_t p0 = (int64_t)si.x * num_heads + head;     // part p sits at p0 + p * num_heads
#pragma unroll 2
            for (int p = pl; p < nparts; p += PL) {
                const int64_t pi = p0 + (int64_t)p * num_heads;
                const float mp = ws_m[pi], lp = ws_l[pi];
                const f32x4 op = *(const f32x4 *)(ws_o + pi * D + 4 * dg);
                const float mn = fmaxf(mm, mp);
                const float a = fast_exp2(mm - mn), w = fast_exp2(mp - mn);
                ll = ll * a + lp * w;
                oo = oo * a + op * w;
                mm = mn;
            }
        }
        s_o[slot][dg] = oo;
        if (dg == 0) {
            s_l[slot] = ll;
            s_m[slot] = mm;
        }
        __syncthreads();
        if (pl == 0 && active) {
            for (int q = 1; q < PL; ++q) {
                const float mq = s_m[slot + q], mn = fmaxf(mm, mq);
                const float a = fast_exp2(mm - mn), w = fast_exp2(mq - mn);
                oo = oo * a + s_o[slot + q][dg] * w;
                ll = ll * a + s_l[slot + q] * w;
                mm = mn;
            }
            const float inv = 1.0f / ll;
            const int64_t o = ((int64_t)seq * num_heads + head) * D + 4 * dg;
            if constexpr (BF16) {
                *(uint2 *)((uint16_t *)out + o) = make_uint2(pack_bf16x2(oo[0] * inv, oo[1] * inv),
                                                             pack_bf16x2(oo[2] * inv, oo[3] * inv));
            } else {
                *(f32x4 *)((float *)out + o) = oo * inv;
            }
        }
        __syncthreads();                        // s_o, s_l, s_m are rewritten by the next entry
    }
}

// The plan kernel, sizing parts for the resident waves of the decode kernel that will run: the matrix-core
// kernel runs one workgroup of DECODE_CU_WAVES_BF16 / _Q8 waves per compute unit, the other a.workers.
// With a decode step's store (a.st_chunks > 0) the plan shares its launch with the store's pieces.
static hipError_t launch_plan(const DecodeArgs &a, bool mfma, bool q8, hipStream_t stream) {
    const int workers = mfma ? a.compute_units * (q8 ? DECODE_CU_WAVES_Q8 : DECODE_CU_WAVES_BF16) : a.workers;
    if (a.st_chunks > 0) {
        const int64_t rows = a.st_tokens * a.num_kv_heads, pieces = rows * a.st_chunks;
        const dim3 grid((unsigned)(1 + (pieces + PLAN_THREADS - 1) / PLAN_THREADS));
        auto k = (const u32x4 *)a.st_key, v = (const u32x4 *)a.st_value;
        auto kc = (u32x4 *)a.st_key_cache, vc = (u32x4 *)a.st_value_cache;
        auto kern = a.st_chunks == 8 ? store_and_plan_kernel<8> : a.st_chunks == 16 ? store_and_plan_kernel<16>
                                                                                   : store_and_plan_kernel<32>;
        if (a.st_chunks != 8 && a.st_chunks != 16 && a.st_chunks != 32) return hipErrorInvalidValue;
        hipLaunchKernelGGL(kern, grid, dim3(PLAN_THREADS), 0, stream, k, v, kc, vc, a.st_slots, rows,
                           a.st_block_size, (int)a.num_blocks, a.context_lens, a.num_seqs, a.max_context_len,
                           a.num_kv_heads, workers, a.min_strata, a.max_part_tiles, a.min_part_tiles, a.items,
                           a.seq_info, a.red_list, a.ctrl, a.key);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, a.context_lens, a.num_seqs,
                       a.max_context_len, a.num_kv_heads, workers, a.min_strata, a.max_part_tiles, a.min_part_tiles,
                       a.items, a.seq_info, a.red_list, a.ctrl, a.key);
    return hipGetLastError();
}

template <bool BF16, int D, int G, int NV, int R, int NW, bool MFMA>
static hipError_t launch_decode_cfg(const DecodeArgs &a, hipStream_t stream) {
    const bool q8 = a.key_scale != nullptr;
    const int nwv = q8 ? DECODE_CU_WAVES_Q8 : DECODE_CU_WAVES_BF16;
    hipError_t e = hipSuccess;
    if (!a.run_only) {
        e = launch_plan(a, MFMA, q8, stream);
        if (e != hipSuccess) return e;
    }
    const int64_t units = (int64_t)a.max_items * a.num_kv_heads;     // upper bound on the unit count
    if constexpr (MFMA) {
        static_assert(BF16 && D == 128, "matrix-core decode: bf16, head_dim 128");
        // one workgroup of nwv waves per compute unit
        const int64_t need = (units + nwv - 1) / nwv;
        const int64_t grid = need < a.compute_units ? need : a.compute_units;
        auto kernel = !q8            ? decode_mfma_kernel<G, false, false>
                      : a.int4_codes ? decode_mfma_kernel<G, true, false, true>
                      : a.fp8_codes  ? decode_mfma_kernel<G, true, true>
                                     : decode_mfma_kernel<G, true, false>;
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid),
                           dim3(64 * nwv), 0, stream, a.out, a.query, (const char *)a.key_cache, (const char *)a.value_cache,
                           a.block_tables, a.bt_stride, a.items, a.ctrl, a.key, a.num_kv_heads, a.num_blocks, a.log2_bs,
                           a.scale_log2e, a.ws_m, a.ws_l, a.ws_o, a.key_scale, a.value_scale);
    } else {
        hipLaunchKernelGGL((decode_kernel<BF16, D, G, NV, R, NW>), dim3((unsigned)units), dim3(64 * NW), 0, stream,
                           a.out, a.query, (const u32x4 *)a.key_cache, (const u32x4 *)a.value_cache, a.block_tables,
                           a.bt_stride, a.items, a.ctrl, a.key, a.num_kv_heads, a.num_blocks, a.log2_bs, a.scale_log2e,
                           a.ws_m, a.ws_l, a.ws_o);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // heads per reduce workgroup: the fewest (1..8) that keep (head groups) x (sequences) at REDUCE_WGS or
    // more; list entries per column: enough columns that the grid holds about REDUCE_WGS workgroups
    const int num_heads = a.num_kv_heads * G;
    int hpb = 8;
    while (hpb > 1 && (int64_t)((num_heads + hpb - 1) / hpb) * a.num_seqs < REDUCE_WGS) hpb >>= 1;
    const int hgroups = (num_heads + hpb - 1) / hpb;
    const int cols = (int)std::min<int64_t>(a.num_seqs, std::max(1, REDUCE_WGS / hgroups));
    hipLaunchKernelGGL((decode_reduce_kernel<BF16, D>), dim3(hgroups, cols), dim3(REDUCE_THREADS), 0, stream, a.out,
                       a.seq_info, a.red_list, num_heads, hpb, a.ws_m, a.ws_l, a.ws_o, a.ctrl, a.key);
    return hipGetLastError();
}

// Kernel shape per (dtype, head_dim, group): vectors per lane NV, tile depth R, waves per workgroup NW.
#ifndef PKV_DECODE_NW
#define PKV_DECODE_NW 1
#endif
#ifndef PKV_DECODE_MFMA_MIN_G
#define PKV_DECODE_MFMA_MIN_G 1  // bf16 head_dim 128 with at least this many query heads per kv head: MFMA
#endif
#ifndef PKV_DECODE_R2
#define PKV_DECODE_R2 2      // tile depth when a lane holds two vectors of a row
#endif
template <bool BF16, int D, int G>
static hipError_t launch_decode_t(const DecodeArgs &a, hipStream_t stream) {
    constexpr int VPR = D / (BF16 ? 8 : 4);
    constexpr int NV = (VPR / ((G <= 4) ? 2 : 1) > 16) ? VPR / 16 : ((G <= 4) ? 2 : 1);
    constexpr int R = (NV == 1) ? 2 * PKV_DECODE_R2 : (NV == 2 ? PKV_DECODE_R2 : 1);
    if constexpr (BF16 && D == 128 && G >= PKV_DECODE_MFMA_MIN_G) {
        if (a.log2_bs >= 4) return launch_decode_cfg<BF16, D, G, NV, R, PKV_DECODE_NW, true>(a, stream);
    }
    return launch_decode_cfg<BF16, D, G, NV, R, PKV_DECODE_NW, false>(a, stream);
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

hipError_t launch_decode_q8(const DecodeArgs &a, int group, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    if (a.log2_bs < 4 || a.key_scale == nullptr || a.value_scale == nullptr) return hipErrorInvalidValue;
    switch (group) {
        case 1: return launch_decode_cfg<true, 128, 1, 2, 2, 1, true>(a, stream);
        case 2: return launch_decode_cfg<true, 128, 2, 2, 2, 1, true>(a, stream);
        case 3: return launch_decode_cfg<true, 128, 3, 2, 2, 1, true>(a, stream);
        case 4: return launch_decode_cfg<true, 128, 4, 2, 2, 1, true>(a, stream);
        case 5: return launch_decode_cfg<true, 128, 5, 1, 4, 1, true>(a, stream);
        case 6: return launch_decode_cfg<true, 128, 6, 1, 4, 1, true>(a, stream);
        case 7: return launch_decode_cfg<true, 128, 7, 1, 4, 1, true>(a, stream);
        case 8: return launch_decode_cfg<true, 128, 8, 1, 4, 1, true>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

bool decode_uses_mfma(bool bf16, int head_dim, int group, int log2_bs) {
    return bf16 && head_dim == 128 && group >= PKV_DECODE_MFMA_MIN_G && group <= 16 && log2_bs >= 4;
}

hipError_t launch_decode_plan(const DecodeArgs &a, bool mfma, bool q8, hipStream_t stream) {
    if (a.num_seqs == 0) return hipSuccess;
    return launch_plan(a, mfma, q8, stream);
}

int decode_max_part_blocks() { return MAX_PART_BLOCKS; }
int decode_tile_tokens() { return DECODE_TILE; }

}  // namespace pkv
