// Host-side KV block manager: fixed-size blocks handed out from a pool, per-request block tables,
// slot mapping for new tokens, usage metrics, and (optionally) prefix caching with copy-on-write.
//
// Behaviour follows the pages:
//  - "LLM Infra 101 v0.5" (ifuryst.com), section KV Block Manager: a FIFO free list; allocate(request,
//    tokens) takes ceil(tokens / block_size) blocks from its front, append grows a request by the blocks
//    its new token count needs, release returns a request's blocks to the back; bad requests and
//    over-allocation are errors; section 推理: block usage (allocated tokens, reserved tokens, internal
//    fragmentation, utilization, used / free blocks) and the contiguous fixed-slot baseline.
//  - nano-vllm walkthrough (lpnh.cn), section 3 Block / BlockManager: blocks carry a reference count and,
//    once full, a chained hash h_i = hash(h_{i-1}, tokens of block i) with its token ids; allocation
//    reuses a block on a hash hit whose token ids match, and after the first miss every later block
//    misses; release walks the table backwards and frees a block when its count reaches zero, keeping
//    its hash; a decode step opens a new block when len % block_size == 1 and registers the hash of a
//    block when it becomes full (len % block_size == 0).
//  - "推理运行时" (wineandchord.com), section Prefix cache 与 copy-on-write: branches share read-only
//    blocks; writing into a shared block that is not full first copies it.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <deque>
#include <memory>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/pagedkv.h"
#include "../../include/pagedkv_blocks.h"

namespace {

thread_local std::string g_bm_err;

pkv_status bm_fail(pkv_status st, const std::string &msg) {
    g_bm_err = msg;
    return st;
}

struct Block {
    int32_t ref = 0;
    bool hashed = false;
    uint64_t hash = 0;
    std::vector<int32_t> tokens;     // token ids of a hashed (full) block
};

struct Request {
    std::vector<int32_t> blocks;
    int64_t num_tokens = 0;
    int64_t num_cached_tokens = 0;
    std::vector<int32_t> token_ids;  // kept only with prefix caching
};

// 64-bit FNV-1a over the previous hash and the block's token ids (a chained hash of the prefix).
uint64_t chain_hash(uint64_t prev, const int32_t *tok, int32_t n) {
    uint64_t h = 1469598103934665603ull;
    auto mix = [&](uint64_t v) {
        for (int b = 0; b < 8; ++b) {
            h ^= (v >> (8 * b)) & 0xffu;
            h *= 1099511628211ull;
        }
    };
    mix(prev);
    for (int32_t i = 0; i < n; ++i) mix((uint64_t)(uint32_t)tok[i]);
    return h;
}

}  // namespace

struct pkv_block_manager {
    int32_t total = 0, bs = 0;
    bool prefix = false;
    std::vector<Block> blocks;
    std::deque<int32_t> free_ids;
    std::unordered_map<uint64_t, int32_t> hash_to_block;
    std::unordered_map<int64_t, Request> reqs;
    std::vector<int32_t> copies;     // pending copy-on-write pairs (src, dst)

    int64_t blocks_for(int64_t tokens) const { return (tokens + bs - 1) / bs; }

    int32_t take_block() {           // caller checked free_ids is non-empty
        int32_t id = free_ids.front();
        free_ids.pop_front();
        Block &b = blocks[id];
        if (b.hashed) {              // recycled: its cached content is about to be overwritten
            auto it = hash_to_block.find(b.hash);
            if (it != hash_to_block.end() && it->second == id) hash_to_block.erase(it);
            b.hashed = false;
            b.tokens.clear();
        }
        b.ref = 1;
        return id;
    }

    void unref(int32_t id) {
        Block &b = blocks[id];
        if (--b.ref == 0) free_ids.push_back(id);
    }

    void register_full(Request &r, int64_t block_index) {
        int32_t id = r.blocks[block_index];
        Block &b = blocks[id];
        uint64_t prev = block_index > 0 ? blocks[r.blocks[block_index - 1]].hash : 0;
        const int32_t *tok = r.token_ids.data() + block_index * bs;
        b.hash = chain_hash(prev, tok, bs);
        b.hashed = true;
        b.tokens.assign(tok, tok + bs);
        hash_to_block[b.hash] = id;
    }
};

extern "C" {

const char *pkv_bm_last_error(void) { return g_bm_err.c_str(); }

pkv_status pkv_bm_create(int32_t total_blocks, int32_t block_size, int32_t prefix_caching, pkv_block_manager **out) {
    if (!out) return bm_fail(PKV_EINVAL, "null output handle");
    *out = nullptr;
    if (total_blocks < 1) return bm_fail(PKV_EINVAL, "total_blocks must be at least 1");
    if (block_size < 1) return bm_fail(PKV_EINVAL, "block_size must be at least 1");
    auto *bm = new (std::nothrow) pkv_block_manager();
    if (!bm) return bm_fail(PKV_ENOMEM, "out of host memory");
    bm->total = total_blocks;
    bm->bs = block_size;
    bm->prefix = prefix_caching != 0;
    bm->blocks.resize(total_blocks);
    for (int32_t i = 0; i < total_blocks; ++i) bm->free_ids.push_back(i);
    *out = bm;
    return PKV_OK;
}

void pkv_bm_destroy(pkv_block_manager *bm) { delete bm; }

pkv_status pkv_bm_allocate(pkv_block_manager *bm, int64_t request_id, int32_t num_tokens, const int32_t *token_ids,
                           int32_t *num_cached_tokens) {
    if (!bm) return bm_fail(PKV_EINVAL, "null block manager");
    if (bm->reqs.count(request_id)) return bm_fail(PKV_EINVAL, "request already has allocated blocks: " + std::to_string(request_id));
    if (num_tokens < 0) return bm_fail(PKV_EINVAL, "token_count must be non-negative");
    if (bm->prefix && num_tokens > 0 && !token_ids) return bm_fail(PKV_EINVAL, "prefix caching needs the token ids");
    const int64_t need = bm->blocks_for(num_tokens);
    Request r;
    r.num_tokens = num_tokens;
    if (bm->prefix) r.token_ids.assign(token_ids, token_ids + num_tokens);
    // prefix cache: reuse full blocks whose chained hash and token ids match, until the first miss
    std::vector<int32_t> hits;
    if (bm->prefix) {
        uint64_t h = 0;
        for (int64_t j = 0; (j + 1) * bm->bs <= num_tokens; ++j) {
            h = chain_hash(h, token_ids + j * bm->bs, bm->bs);
            auto it = bm->hash_to_block.find(h);
            if (it == bm->hash_to_block.end()) break;
            const Block &b = bm->blocks[it->second];
            if (!std::equal(b.tokens.begin(), b.tokens.end(), token_ids + j * bm->bs)) break;
            hits.push_back(it->second);
        }
    }
    // a hit on a freed block takes it back out of the free list
    int64_t hits_free = 0;
    for (int32_t id : hits) hits_free += bm->blocks[id].ref == 0;
    const int64_t fresh = need - (int64_t)hits.size();
    if (fresh > (int64_t)bm->free_ids.size() - hits_free)
        return bm_fail(PKV_ENOMEM, "not enough free blocks: need " + std::to_string(fresh) + ", have " +
                                      std::to_string((int64_t)bm->free_ids.size() - hits_free));
    for (int32_t id : hits) {
        Block &b = bm->blocks[id];
        if (b.ref == 0) bm->free_ids.erase(std::find(bm->free_ids.begin(), bm->free_ids.end(), id));
        b.ref += 1;
        r.blocks.push_back(id);
    }
    r.num_cached_tokens = (int64_t)hits.size() * bm->bs;
    for (int64_t j = (int64_t)hits.size(); j < need; ++j) r.blocks.push_back(bm->take_block());
    if (bm->prefix)
        for (int64_t j = (int64_t)hits.size(); (j + 1) * bm->bs <= num_tokens; ++j) bm->register_full(r, j);
    if (num_cached_tokens) *num_cached_tokens = (int32_t)r.num_cached_tokens;
    bm->reqs.emplace(request_id, std::move(r));
    return PKV_OK;
}

pkv_status pkv_bm_append(pkv_block_manager *bm, int64_t request_id, int32_t num_tokens, const int32_t *token_ids) {
    if (!bm) return bm_fail(PKV_EINVAL, "null block manager");
    if (num_tokens < 0) return bm_fail(PKV_EINVAL, "token_count must be non-negative");
    auto it = bm->reqs.find(request_id);
    if (it == bm->reqs.end()) return bm_fail(PKV_EINVAL, "request has no allocated blocks: " + std::to_string(request_id));
    if (num_tokens == 0) return PKV_OK;
    if (bm->prefix && !token_ids) return bm_fail(PKV_EINVAL, "prefix caching needs the token ids");
    Request &r = it->second;
    const int64_t old_tokens = r.num_tokens, new_tokens = old_tokens + num_tokens;
    const int64_t extra = bm->blocks_for(new_tokens) - bm->blocks_for(old_tokens);
    // copy-on-write: the partial last block is shared and this append writes into it
    const bool cow = old_tokens % bm->bs != 0 && !r.blocks.empty() && bm->blocks[r.blocks.back()].ref > 1;
    if (extra + (cow ? 1 : 0) > (int64_t)bm->free_ids.size())
        return bm_fail(PKV_ENOMEM, "not enough free blocks: need " + std::to_string(extra + (cow ? 1 : 0)) + ", have " +
                                      std::to_string(bm->free_ids.size()));
    if (cow) {
        const int32_t src = r.blocks.back();
        const int32_t dst = bm->take_block();
        bm->unref(src);
        r.blocks.back() = dst;
        bm->copies.push_back(src);
        bm->copies.push_back(dst);
    }
    for (int64_t j = 0; j < extra; ++j) r.blocks.push_back(bm->take_block());
    if (bm->prefix) r.token_ids.insert(r.token_ids.end(), token_ids, token_ids + num_tokens);
    r.num_tokens = new_tokens;
    if (bm->prefix)
        for (int64_t j = old_tokens / bm->bs; (j + 1) * bm->bs <= new_tokens; ++j) bm->register_full(r, j);
    return PKV_OK;
}

pkv_status pkv_bm_fork(pkv_block_manager *bm, int64_t parent_id, int64_t child_id) {
    if (!bm) return bm_fail(PKV_EINVAL, "null block manager");
    auto it = bm->reqs.find(parent_id);
    if (it == bm->reqs.end()) return bm_fail(PKV_EINVAL, "request has no allocated blocks: " + std::to_string(parent_id));
    if (bm->reqs.count(child_id)) return bm_fail(PKV_EINVAL, "request already has allocated blocks: " + std::to_string(child_id));
    Request child = it->second;
    for (int32_t id : child.blocks) bm->blocks[id].ref += 1;
    child.num_cached_tokens = child.num_tokens;
    bm->reqs.emplace(child_id, std::move(child));
    return PKV_OK;
}

pkv_status pkv_bm_release(pkv_block_manager *bm, int64_t request_id) {
    if (!bm) return bm_fail(PKV_EINVAL, "null block manager");
    auto it = bm->reqs.find(request_id);
    if (it == bm->reqs.end()) return bm_fail(PKV_EINVAL, "request has no allocated blocks: " + std::to_string(request_id));
    const std::vector<int32_t> &b = it->second.blocks;
    for (auto rit = b.rbegin(); rit != b.rend(); ++rit) bm->unref(*rit);   // last block first
    bm->reqs.erase(it);
    return PKV_OK;
}

pkv_status pkv_bm_block_table(const pkv_block_manager *bm, int64_t request_id, int32_t *out, int32_t capacity,
                              int32_t *num_blocks, int64_t *num_tokens) {
    if (!bm) return bm_fail(PKV_EINVAL, "null block manager");
    auto it = bm->reqs.find(request_id);
    if (it == bm->reqs.end()) return bm_fail(PKV_EINVAL, "request has no allocated blocks: " + std::to_string(request_id));
    const Request &r = it->second;
    if (num_blocks) *num_blocks = (int32_t)r.blocks.size();
    if (num_tokens) *num_tokens = r.num_tokens;
    if (out) {
        if (capacity < (int32_t)r.blocks.size()) return bm_fail(PKV_EINVAL, "block table buffer too small");
        for (size_t j = 0; j < r.blocks.size(); ++j) out[j] = r.blocks[j];
        for (int32_t j = (int32_t)r.blocks.size(); j < capacity; ++j) out[j] = -1;
    }
    return PKV_OK;
}

pkv_status pkv_bm_slot_mapping(const pkv_block_manager *bm, int64_t request_id, int64_t first_position, int32_t count,
                               int32_t *slots) {
    if (!bm) return bm_fail(PKV_EINVAL, "null block manager");
    auto it = bm->reqs.find(request_id);
    if (it == bm->reqs.end()) return bm_fail(PKV_EINVAL, "request has no allocated blocks: " + std::to_string(request_id));
    const Request &r = it->second;
    if (count < 0 || first_position < 0 || first_position + count > r.num_tokens)
        return bm_fail(PKV_EINVAL, "positions outside the request's tokens");
    if (count > 0 && !slots) return bm_fail(PKV_EINVAL, "null slots");
    for (int32_t k = 0; k < count; ++k) {
        const int64_t pos = first_position + k;
        slots[k] = r.blocks[pos / bm->bs] * bm->bs + (int32_t)(pos % bm->bs);
    }
    return PKV_OK;
}

pkv_status pkv_bm_take_copies(pkv_block_manager *bm, int32_t *pairs, int32_t capacity, int32_t *num_pairs) {
    if (!bm || !num_pairs) return bm_fail(PKV_EINVAL, "null argument");
    const int32_t n = (int32_t)(bm->copies.size() / 2);
    *num_pairs = n;
    if (!pairs) return PKV_OK;                        // query only
    if (capacity < n) return bm_fail(PKV_EINVAL, "copy list buffer too small");
    std::copy(bm->copies.begin(), bm->copies.end(), pairs);
    bm->copies.clear();
    return PKV_OK;
}

pkv_status pkv_bm_usage(const pkv_block_manager *bm, pkv_bm_usage_t *u) {
    if (!bm || !u) return bm_fail(PKV_EINVAL, "null argument");
    memset(u, 0, sizeof *u);
    int64_t used = 0;
    for (const Block &b : bm->blocks) used += b.ref > 0;
    for (const auto &kv : bm->reqs) {
        u->allocated_tokens += kv.second.num_tokens;
        u->max_request_tokens = std::max(u->max_request_tokens, kv.second.num_tokens);
    }
    u->num_requests = (int64_t)bm->reqs.size();
    u->used_blocks = used;
    u->free_blocks = (int64_t)bm->free_ids.size();
    u->reserved_tokens = used * bm->bs;
    u->internal_fragmentation_tokens = u->reserved_tokens - u->allocated_tokens;
    u->block_utilization = u->reserved_tokens ? (double)u->allocated_tokens / (double)u->reserved_tokens : 0.0;
    u->contiguous_reserved_tokens = u->num_requests * u->max_request_tokens;
    u->contiguous_fragmentation_tokens = u->contiguous_reserved_tokens - u->allocated_tokens;
    u->contiguous_utilization =
        u->contiguous_reserved_tokens ? (double)u->allocated_tokens / (double)u->contiguous_reserved_tokens : 0.0;
    return PKV_OK;
}

}  // extern "C"
