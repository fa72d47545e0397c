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
// Work decomposition. One workgroup per (sequence, kv head, query tile). Workgroups are dealt to the
// 8 XCDs round-robin by their linear id, so the id is remapped to keep every query tile of one
// (sequence, kv head) on the same XCD, dispatched back to back (the heaviest, last tile first): the
// K/V rows they all read then come from that XCD's L2 instead of being fetched once per tile.
// A 256-thread workgroup (4 waves) owns
// 128 "rows" = BQ query positions x the G query heads that share the kv head (row = pos * G + h),
// so each K/V tile brought into LDS serves all G heads. Each wave owns 32 rows. The key loop walks
// 64-key tiles up to the last key any row of the tile may see; the next tile's K/V rows are loaded
// into registers while the current tile is computed.
//   - Gather: K and V rows both go to LDS row-major (16-byte stores, no transposition in registers).
//   - S^T = K Q^T on MFMA: K (LDS) is the A operand, Q (registers) the B operand. In the 16x16
//     output block lane l holds keys 4*(l/16)+i of query row l%16.
//   - Mask (causal, bottom-right aligned; sequence end), online softmax per query row in log2 units:
//     a row's 64 scores sit in 16 values of each of 4 lanes (lane, lane^16, lane^32, lane^48).
//   - O^T += V^T P^T on MFMA: the rounded weights of S^T's registers are already laid out as the B
//     operand (a lane's 8 reduction elements are keys {4b..4b+3} and {16+4b..16+4b+3} of a 32-key
//     step, b = l/16), and V^T comes out of the row-major V tile through ds_read_b64_tr_b16, the
//     gfx950 transposing LDS read (in a 16-lane group, lane i receives element i % 4 of the 8-byte
//     chunks read by lanes 4k + i / 4, k = 0..3), in the same key order. P never goes through LDS.
// The MFMA output layout is the 16x16 fp32 block with lane l holding rows 4*(l/16)+i, column l%16;
// the A/B operands take 8 reduction elements per lane, paired between the operands element by
// element, so any reduction order of the hardware sums matching pairs.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace pkv {


constexpr int PF_THREADS = 256;
constexpr int PF_D = 128;
constexpr int PF_BN = 64;                 // keys per tile
constexpr int PF_KPAD = PF_D + 16;        // LDS row stride of the K and V tiles, bf16 elements (288 bytes)
constexpr float PF_M_INIT = -1.0e30f;
constexpr float PF_RESCALE_SLACK = 8.0f;  // weights stay <= 256 between rescales
constexpr int PF_RANK_MAX = 64;           // batches ranked by length for the dispatch order
constexpr int PF_XCDS = 8;                // MI355X: 8 XCDs, each with its own L2
constexpr int PF_BUF_W3 = 0x00020000;     // buffer descriptor word 3: raw, untyped buffer (gfx9 family)
constexpr int PF_KAHEAD = 4;              // K operand reads in flight ahead of the S^T MFMAs
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int SGB_MFMA = 0x008, SGB_DS_READ = 0x100;

typedef short i16x4 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16 at an LDS address (8 bytes, 8-byte aligned), as two dwords.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t *p) {
    const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)p);
    return __builtin_bit_cast(u32x2, v);
}

// QB: 16-row blocks per wave (rows per wave 16 QB, per workgroup 64 QB). Every K and V^T value read from
// LDS feeds QB MFMAs, so LDS traffic per MFMA falls as QB grows; QB = 4 takes one wave per SIMD.
//
// 8-bit caches (Q8): rows hold one-byte codes (int8, or OCP float8 E4M3 when F8) with one fp32 scale per
// (token, kv head). The gather loads the codes and the tile's 64 key and 64 value scales; codes become exact
// bf16 values as the tile is stored to LDS, so the rest of the tile's work is the bf16 path's. The K scale
// multiplies each score (before the mask), and the V scale each weight before it is rounded to bf16; the
// denominator sums the unscaled weights (so out = sum_t p_t v_t scale_t / sum_t p_t, the attention over the
// dequantized rows).
template <bool F8, int K>
__device__ __forceinline__ uint32_t pf_code_pair_to_bf16x2(uint32_t w) {
    if constexpr (F8) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, K != 0));
    else return i8pair_to_bf16x2(w, K);
}
// 16 codes -> 16 bf16 values in order (two 16-byte LDS stores)
template <bool F8>
__device__ __forceinline__ void pf_codes_to_bf16(const u32x4 c, u32x4 &lo, u32x4 &hi) {
    lo = u32x4{pf_code_pair_to_bf16x2<F8, 0>(c[0]), pf_code_pair_to_bf16x2<F8, 1>(c[0]),
               pf_code_pair_to_bf16x2<F8, 0>(c[1]), pf_code_pair_to_bf16x2<F8, 1>(c[1])};
    hi = u32x4{pf_code_pair_to_bf16x2<F8, 0>(c[2]), pf_code_pair_to_bf16x2<F8, 1>(c[2]),
               pf_code_pair_to_bf16x2<F8, 0>(c[3]), pf_code_pair_to_bf16x2<F8, 1>(c[3])};
}

template <int G, int QB, bool Q8 = false, bool F8 = false>
__global__ void __launch_bounds__(PF_THREADS) __attribute__((amdgpu_waves_per_eu(QB <= 2 ? 2 : 1, QB <= 2 ? 2 : 1)))
prefill_kernel(uint16_t *__restrict__ out, const u32x4 *__restrict__ query, const u32x4 *__restrict__ key_cache,
               const u32x4 *__restrict__ value_cache, const int32_t *__restrict__ block_tables, int bt_stride,
               const int32_t *__restrict__ cu_seqlens_q, const int32_t *__restrict__ cu_seqlens_k, int num_seqs,
               int max_seqlen_k, int num_q_tiles, int num_kv_heads, int64_t num_blocks, int log2_bs, float scale_log2e,
               int causal, const float *__restrict__ key_scale = nullptr, const float *__restrict__ value_scale = nullptr) {
    constexpr int WROWS = 16 * QB;            // rows per wave
    constexpr int ROWS = 4 * WROWS;           // rows per workgroup
    constexpr int BQ = ROWS / G;              // query positions per workgroup
    constexpr int VR = BQ * G;                // rows in use (<= ROWS)
    constexpr int CH = PF_D / 8;              // 16-byte chunks per bf16 row (query, LDS tiles)
    constexpr int RCH = Q8 ? PF_D / 16 : CH;  // 16-byte chunks per cache row
    constexpr int NC = PF_BN * RCH / PF_THREADS;   // cache chunks of a tile per thread (K, and V): 4 or 2

    __shared__ __attribute__((aligned(16))) uint16_t sK[2][PF_BN * PF_KPAD];     // double-buffered tiles
    __shared__ __attribute__((aligned(16))) uint16_t sV[2][PF_BN * PF_KPAD];
    __shared__ __attribute__((aligned(16))) float sS[2][2][Q8 ? PF_BN : 1];         // [buf][K, V][key] scales

    // linear id w runs on XCD w % 8: group g = (sequence rank, kv head) lives on XCD g % 8
    const int w = blockIdx.x, xcd = w & (PF_XCDS - 1), j = w / PF_XCDS;
    // (divisions run on the vector ALU; readfirstlane states that the results are wave-uniform, so
    // addresses built from them stay in scalar registers)
    const int g = __builtin_amdgcn_readfirstlane((j / num_q_tiles) * PF_XCDS + xcd);
    if (g >= num_seqs * num_kv_heads) return;
    const int qt = __builtin_amdgcn_readfirstlane(num_q_tiles - 1 - j % num_q_tiles);
    const int rank = __builtin_amdgcn_readfirstlane(g / num_kv_heads), kvh = __builtin_amdgcn_readfirstlane(g % num_kv_heads);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Dispatch order: workgroups start in linear-id order, and the sequence of rank r is the r-th longest
    // (most keys; ties by index), so the longest work starts first and short work fills the tail. Each
    // workgroup ranks the batch itself, one thread per sequence (batches of up to PF_RANK_MAX sequences;
    // larger ones keep their order).
    int seq = rank;
    if (num_seqs > 1 && num_seqs <= PF_RANK_MAX) {
        __shared__ int s_len[PF_RANK_MAX];
        __shared__ int s_seq;
        int lk = 0;
        if (tid < num_seqs) {
            lk = cu_seqlens_k[tid + 1] - cu_seqlens_k[tid];
            s_len[tid] = lk;
        }
        __syncthreads();
        if (tid < num_seqs) {
            int r = 0;
            for (int u = 0; u < num_seqs; ++u) {
                const int lu = s_len[u];
                r += (lu > lk) | ((lu == lk) & (u < tid));
            }
            if (r == rank) s_seq = tid;                     // ranks are a permutation: one thread writes
        }
        __syncthreads();
        seq = s_seq;
    }
    seq = __builtin_amdgcn_readfirstlane(seq);
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
    const int kfull = causal ? P + pos0 + 1 : Lk;              // keys [0, kfull) visible to every row
    const int bs_mask = (1 << log2_bs) - 1;
    const int32_t *bt = block_tables + (int64_t)seq * bt_stride;

    // this lane's QB query rows (one per 16-row block qb): row = wave * WROWS + 16*qb + lr
    int kmax[QB];
    bool row_ok[QB];
    u32x4 qb_reg[QB][4];                      // B operand of S^T: dims 8*lb + 32*ks .. +8 of the row
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int r = wave * WROWS + qb * 16 + lr;
        const int pos = r / G, h = r % G;
        row_ok[qb] = r < VR && pos < npos;
        kmax[qb] = causal ? P + pos0 + pos : Lk - 1;
        const int64_t qrow = ((int64_t)(q0 + pos0 + (row_ok[qb] ? pos : 0)) * num_heads + kvh * G + h) * CH;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qb_reg[qb][ks] = row_ok[qb] ? query[qrow + lb + 4 * ks] : u32x4{0, 0, 0, 0};
    }

    // gather roles: thread tid moves 16-byte cache chunks tid + 256 c (c < NC) of the K and of the V tile;
    // over 8-bit caches threads 0..63 also move the key scale of key tid, threads 64..127 the value scale
    u32x4 kreg[NC], vreg[NC];
    float sreg = 0.f;
    // the first 64 block ids of the sequence, one per lane (uniform tiles read them with readlane)
    const int nblk_seq = (Lk + bs_mask) >> log2_bs;
    const int my_blk = lane < nblk_seq ? bt[lane] : -1;
    auto load_tile = [&](int key0) {
        if (log2_bs >= 6 && key0 + PF_BN <= kend) {
            // The whole tile lies in one block (64 | block_size, tiles start at multiples of 64): one buffer
            // descriptor for the (block, kv head) slab, the tile's row as scalar offset, lane offsets fixed.
            // A block id outside the pool gets an empty descriptor, whose loads return zeros.
            const int j = key0 >> log2_bs;
            // (readfirstlane: the id is wave-uniform; saying so keeps the descriptor in scalar registers)
            const int64_t blk = __builtin_amdgcn_readfirstlane(j < 64 ? __builtin_amdgcn_readlane(my_blk, j) : bt[j]);
            const bool ok = blk >= 0 && blk < num_blocks;
            const int64_t slab = ((ok ? blk : 0) * num_kv_heads + kvh) << log2_bs;       // first row
            const int range = ok ? (int)((uint32_t)RCH * 16u << log2_bs) : 0;
            const __amdgpu_buffer_rsrc_t kr =
                __builtin_amdgcn_make_buffer_rsrc((void *)(key_cache + slab * RCH), (short)0, range, PF_BUF_W3);
            const __amdgpu_buffer_rsrc_t vr =
                __builtin_amdgcn_make_buffer_rsrc((void *)(value_cache + slab * RCH), (short)0, range, PF_BUF_W3);
            const int soff = (key0 & bs_mask) * RCH * 16;
#pragma unroll
            for (int c = 0; c < NC; ++c)
                kreg[c] = __builtin_amdgcn_raw_buffer_load_b128(kr, (tid + c * PF_THREADS) * 16, soff, 0);
#pragma unroll
            for (int c = 0; c < NC; ++c)
                vreg[c] = __builtin_amdgcn_raw_buffer_load_b128(vr, (tid + c * PF_THREADS) * 16, soff, 0);
            if constexpr (Q8) {
                if (tid < 2 * PF_BN) {
                    const float *sc = tid < PF_BN ? key_scale : value_scale;
                    sreg = ok ? sc[slab + (key0 & bs_mask) + (tid & (PF_BN - 1))] : 0.f;
                }
            }
            return;
        }
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int idx = tid + c * PF_THREADS;
            const int gk = key0 + idx / RCH, ch = idx % RCH;
            kreg[c] = vreg[c] = u32x4{0, 0, 0, 0};
            if (gk < kend) {
                const int64_t blk = bt[gk >> log2_bs];
                if (blk >= 0 && blk < num_blocks) {
                    const int64_t row = ((blk * num_kv_heads + kvh) << log2_bs) + (gk & bs_mask);
                    kreg[c] = key_cache[row * RCH + ch];
                    vreg[c] = value_cache[row * RCH + ch];
                }
            }
        }
        if constexpr (Q8) {                     // scales of keys past the end or outside the pool: 0
            sreg = 0.f;
            const int gk = key0 + (tid & (PF_BN - 1));
            if (tid < 2 * PF_BN && gk < kend) {
                const int64_t blk = bt[gk >> log2_bs];
                if (blk >= 0 && blk < num_blocks)
                    sreg = (tid < PF_BN ? key_scale : value_scale)[((blk * num_kv_heads + kvh) << log2_bs) + (gk & bs_mask)];
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int idx = tid + c * PF_THREADS;
            if constexpr (Q8) {                  // 16 codes -> dims 16 ch .. +16 of the row, as bf16
                u32x4 lo, hi;
                uint16_t *kp = &sK[buf][(idx / RCH) * PF_KPAD + (idx % RCH) * 16];
                uint16_t *vp = &sV[buf][(idx / RCH) * PF_KPAD + (idx % RCH) * 16];
                pf_codes_to_bf16<F8>(kreg[c], lo, hi);
                *(u32x4 *)kp = lo;
                *(u32x4 *)(kp + 8) = hi;
                pf_codes_to_bf16<F8>(vreg[c], lo, hi);
                *(u32x4 *)vp = lo;
                *(u32x4 *)(vp + 8) = hi;
            } else {
                *(u32x4 *)&sK[buf][(idx / CH) * PF_KPAD + (idx % CH) * 8] = kreg[c];
                *(u32x4 *)&sV[buf][(idx / CH) * PF_KPAD + (idx % CH) * 8] = vreg[c];
            }
        }
        if constexpr (Q8) {
            if (tid < 2 * PF_BN) sS[buf][tid / PF_BN][tid & (PF_BN - 1)] = sreg;
        }
    };

    f32x4 o[8][QB];                           // O^T blocks: dims 16*db + 4*lb + i, row 16*qb + lr
    float m[QB], l[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < 8; ++db) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[qb] = PF_M_INIT;
        l[qb] = 0.f;
    }

    load_tile(0);
    store_tile(0);
    __syncthreads();
    // One tile: load the next, Sᵀ, (mask), softmax, Oᵀ += VᵀPᵀ, store the next. MASKED is a compile-time
    // flag: tiles wholly below every row's causal bound and the sequence end (the first nfull) run a body
    // with no mask code at all.
    auto tile_step = [&](int kt, auto masked_flag) {
        constexpr bool MASKED = decltype(masked_flag)::value;
        const int key0 = kt * PF_BN, cur = kt & 1;
        if (kt + 1 < ntiles) load_tile(key0 + PF_BN);      // in flight during this tile's math

        // S^T = K Q^T: s[kb][qb] holds keys 16*kb + 4*lb + i of row 16*qb + lr. The 16 K operands (step
        // t = 4 kb + ks) are read PF_KAHEAD steps ahead of the MFMAs that take them; the scheduling groups
        // below keep that order (left alone, the compiler waits on every second read).
        f32x4 s[4][QB];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        {
            u32x4 ka[PF_KAHEAD];
            auto kread = [&](int t) {
                return *(const u32x4 *)&sK[cur][((t >> 2) * 16 + lr) * PF_KPAD + lb * 8 + (t & 3) * 32];
            };
#pragma unroll
            for (int t = 0; t < PF_KAHEAD; ++t) ka[t] = kread(t);
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                const u32x4 a = ka[t % PF_KAHEAD];
                if (t + PF_KAHEAD < 16) ka[t % PF_KAHEAD] = kread(t + PF_KAHEAD);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[t >> 2][qb] = mfma16x16x32(a, qb_reg[qb][t & 3], s[t >> 2][qb]);
            }
            __builtin_amdgcn_sched_group_barrier(SGB_DS_READ, PF_KAHEAD, 0);
#pragma unroll
            for (int t = 0; t < 16 - PF_KAHEAD; ++t) {
                __builtin_amdgcn_sched_group_barrier(SGB_MFMA, QB, 0);
                __builtin_amdgcn_sched_group_barrier(SGB_DS_READ, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(SGB_MFMA, QB * PF_KAHEAD, 0);
        }

        // 8-bit caches: each score times its key's scale (keys 16 kb + 4 lb + i), before the mask
        f32x4 vsc[4];
        if constexpr (Q8) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const f32x4 ks = *(const f32x4 *)&sS[cur][0][kb * 16 + lb * 4];
                vsc[kb] = *(const f32x4 *)&sS[cur][1][kb * 16 + lb * 4];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[kb][qb] *= ks;
            }
        }
        // mask, online softmax per row, rounded weights packed as the B operand of O^T += V^T P^T
        // (scores stay unscaled until the exponent: scale > 0 keeps the max; m is kept in scaled units)
        if constexpr (MASKED) {                              // some key of this tile is hidden from a row
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = key0 + kb * 16 + lb * 4 + i;
                        if (!(row_ok[qb] && key <= kmax[qb])) s[kb][qb][i] = -INFINITY;
                    }
        }
        float m_new[QB];
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
                mx = fmaxf(fmaxf(mx, fmaxf(s[kb][qb][0], s[kb][qb][1])), fmaxf(s[kb][qb][2], s[kb][qb][3]));
            mx = lane_blocks_max(mx);
            m_new[qb] = fmaxf(m[qb], mx * scale_log2e);
            grow |= m_new[qb] > m[qb] + PF_RESCALE_SLACK;
        }
        // Rescale only when some row's max passes its reference m by more than PF_RESCALE_SLACK (log2 units);
        // otherwise m stays as is, and weights 2^(s - m) reach at most 2^PF_RESCALE_SLACK. The final
        // division by l, summed with the same reference, makes the result independent of m.
        if (__builtin_amdgcn_ballot_w64(grow)) {
            asm volatile("" ::: "memory");                   // a real branch, not speculated multiplies
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float alpha = fast_exp2(m[qb] - m_new[qb]);
                l[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < 8; ++db) o[db][qb] *= alpha;
                m[qb] = m_new[qb];
            }
        }
        u32x4 pb[2][QB];                                     // [ks][qb]
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float nm = -m[qb];
            float rs = 0.f;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                uint32_t w[4];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int kb = 2 * ks + half;
                    if constexpr (Q8) {          // weights times the V scales; the sum takes them unscaled
                        float p[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            p[i] = fast_exp2(fmaf(s[kb][qb][i], scale_log2e, nm));
                            rs += p[i];
                        }
                        w[2 * half] = pack_bf16x2(p[0] * vsc[kb][0], p[1] * vsc[kb][1]);
                        w[2 * half + 1] = pack_bf16x2(p[2] * vsc[kb][2], p[3] * vsc[kb][3]);
                    } else {
                        w[2 * half] = pack_bf16x2(fast_exp2(fmaf(s[kb][qb][0], scale_log2e, nm)),
                                                  fast_exp2(fmaf(s[kb][qb][1], scale_log2e, nm)));
                        w[2 * half + 1] = pack_bf16x2(fast_exp2(fmaf(s[kb][qb][2], scale_log2e, nm)),
                                                      fast_exp2(fmaf(s[kb][qb][3], scale_log2e, nm)));
                    }
                }
                if constexpr (!Q8) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) rs = dot2_bf16(w[e], 0x3f803f80u, rs);   // sum of the rounded weights
                }
                pb[ks][qb] = u32x4{w[0], w[1], w[2], w[3]};
            }
            l[qb] += rs;
        }

        // O^T += V^T P^T: A operand = V^T rows (dims) with keys {4b..4b+3} and {16+4b..16+4b+3} of the step.
        // Lane (lr, b) points its transposing read at key 32 ks + 4 b + lr / 4 (+16 for the second half),
        // dims 16 db + 4 (lr % 4) .. +4; it receives dim 16 db + lr of keys 4b .. 4b + 3 (+16).
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const uint16_t *vp = &sV[cur][(ks * 32 + lb * 4 + (lr >> 2)) * PF_KPAD + db * 16 + 4 * (lr & 3)];
                const u32x2 a0 = lds_read_tr16(vp);
                const u32x2 a1 = lds_read_tr16(vp + 16 * PF_KPAD);
                const u32x4 va = u32x4{a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[db][qb] = mfma16x16x32(va, pb[ks][qb], o[db][qb]);
            }
        }
        // the next tile goes to the other buffer, which every wave finished reading before the last barrier
        if (kt + 1 < ntiles) store_tile(cur ^ 1);
        __syncthreads();            // the next tile is in LDS, and every wave is done with this one
    };
    const int nfull = min(ntiles, kfull / PF_BN);             // tiles with every key visible to every row
    for (int kt = 0; kt < nfull; ++kt) tile_step(kt, std::integral_constant<bool, false>{});
    for (int kt = nfull; kt < ntiles; ++kt) tile_step(kt, std::integral_constant<bool, true>{});

    // normalise and write: lane holds dims 16*db + 4*lb + i of row 16*qb + lr
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float lsum = l[qb];
        lsum += __shfl_xor(lsum, 16);
        lsum += __shfl_xor(lsum, 32);
        const int r = wave * WROWS + qb * 16 + lr;
        const int pos = r / G, h = r % G;
        if (!row_ok[qb]) continue;
        const float inv = 1.0f / lsum;
        uint16_t *orow = out + ((int64_t)(q0 + pos0 + pos) * num_heads + kvh * G + h) * PF_D;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            const u32x2 pk = u32x2{pack_bf16x2(o[db][qb][0] * inv, o[db][qb][1] * inv),
                                   pack_bf16x2(o[db][qb][2] * inv, o[db][qb][3] * inv)};
            *(u32x2 *)&orow[db * 16 + lb * 4] = pk;
        }
    }
}

#ifndef PKV_PREFILL_QB
#define PKV_PREFILL_QB 2
#endif

template <int G, bool Q8 = false, bool F8 = false>
static hipError_t launch_prefill_g(const PrefillArgs &a, hipStream_t stream) {
    constexpr int QB = PKV_PREFILL_QB;
    constexpr int BQ = 64 * QB / G;
    const int num_q_tiles = (a.max_seqlen_q + BQ - 1) / BQ;
    const int64_t groups = (int64_t)a.num_seqs * a.num_kv_heads;
    const int64_t wgs = (groups + PF_XCDS - 1) / PF_XCDS * PF_XCDS * num_q_tiles;
    hipLaunchKernelGGL((prefill_kernel<G, QB, Q8, F8>), dim3((unsigned)wgs), dim3(PF_THREADS), 0, stream,
                       (uint16_t *)a.out, (const u32x4 *)a.query, (const u32x4 *)a.key_cache,
                       (const u32x4 *)a.value_cache, a.block_tables, a.bt_stride, a.cu_seqlens_q, a.cu_seqlens_k,
                       a.num_seqs, a.max_seqlen_k, num_q_tiles, a.num_kv_heads, a.num_blocks, a.log2_bs,
                       a.scale_log2e, a.causal, a.key_scale, a.value_scale);
    return hipGetLastError();
}

template <bool F8>
static hipError_t launch_prefill_q8_f(const PrefillArgs &a, int group, hipStream_t stream) {
    switch (group) {
        case 1: return launch_prefill_g<1, true, F8>(a, stream);
        case 2: return launch_prefill_g<2, true, F8>(a, stream);
        case 3: return launch_prefill_g<3, true, F8>(a, stream);
        case 4: return launch_prefill_g<4, true, F8>(a, stream);
        case 5: return launch_prefill_g<5, true, F8>(a, stream);
        case 6: return launch_prefill_g<6, true, F8>(a, stream);
        case 7: return launch_prefill_g<7, true, F8>(a, stream);
        case 8: return launch_prefill_g<8, true, F8>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_prefill_q8(const PrefillArgs &a, int group, hipStream_t stream) {
    if (a.num_seqs == 0 || a.max_seqlen_q == 0) return hipSuccess;
    if (!a.key_scale || !a.value_scale) return hipErrorInvalidValue;
    return a.fp8_codes ? launch_prefill_q8_f<true>(a, group, stream) : launch_prefill_q8_f<false>(a, group, stream);
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
