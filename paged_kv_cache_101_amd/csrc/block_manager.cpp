// block_manager.cpp -- host-side KV block manager (declared in pkv_blocks.h).
//
// The pool and its policies follow the ttlab page ("Basics of LLM Inference
// and vLLM Internals"): section 4 (block tables, blocks taken one at a time,
// reference-counted sharing with copy-on-write, a doubly linked free queue,
// block 0 reserved as the null block), section 5 (hash chain over full
// blocks, prefix-only hits in whole blocks with the last prompt token always
// recomputed, freed blocks keeping their hashes, consumed from the front of
// the queue and returned tail block first), and sections 9 and 10 (the block
// LRU model: a free block without a cached hash is reused before a cached one
// is evicted).
//
// Data structures:
//  * blocks[]: per physical block its free-queue links (an intrusive doubly
//    linked list, O(1) removal from anywhere), reference count, and -- while
//    it is cached -- its chain hash and the exact content that hash names:
//    its 16 token ids, the extra key and its parent block (id and hand-out
//    generation). A lookup by hash is confirmed against that content, so a
//    hit never depends on the hash being free of collisions.
//  * cache: chain hash -> block, for cached blocks (free or held).
//  * requests: id -> tokens with slots, block table, chain hashes of its full
//    blocks.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv.h"
#include "pkv_blocks.h"

#define PKV_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

constexpr int kBS = PKV_BLOCK_SIZE;

// 64-bit FNV-1a (Fowler, Noll and Vo): the hash of bytes, chained from h.
constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;
uint64_t fnv1a(uint64_t h, const void* data, size_t n) {
    const unsigned char* p = static_cast<const unsigned char*>(data);
    for (size_t i = 0; i < n; ++i) {
        h ^= p[i];
        h *= kFnvPrime;
    }
    return h;
}

// Chain hash of a full block: its parent's chain hash (none for the first
// block), its 16 token ids and the request's extra key.
uint64_t block_hash(bool has_parent, uint64_t parent_hash, const int64_t* tokens, uint64_t extra) {
    uint64_t h = kFnvOffset;
    const unsigned char tag = has_parent ? 1 : 0;
    h = fnv1a(h, &tag, 1);
    h = fnv1a(h, &parent_hash, sizeof parent_hash);
    h = fnv1a(h, tokens, sizeof(int64_t) * kBS);
    h = fnv1a(h, &extra, sizeof extra);
    return h;
}

struct Block {
    int32_t prev = -1, next = -1;  // free-queue links
    bool in_free = false;
    int32_t ref = 0;
    uint32_t gen = 0;              // bumped at every hand-out
    bool cached = false;
    uint64_t hash = 0;
    int32_t parent = -1;           // cached content: parent block (or -1) ...
    uint32_t parent_gen = 0;       // ... as handed out then,
    uint64_t extra = 0;            // the extra key,
    int64_t tokens[kBS];           // and the token ids
};

struct Request {
    std::vector<int64_t> prompt;
    std::vector<int64_t> tokens;   // tokens with slots, in order
    std::vector<int32_t> table;    // physical block of each logical block
    std::vector<uint64_t> chain;   // chain hash of each full block, in order
    uint64_t extra = 0;
};

}  // namespace

struct pkv_block_manager {
    int32_t num_blocks = 0;
    bool caching = false;
    std::vector<Block> blocks;
    int32_t head = -1, tail = -1, nfree = 0;
    std::unordered_map<uint64_t, int32_t> cache;
    std::unordered_map<int64_t, Request> reqs;
    int64_t queried = 0, hit = 0;

    // ---- the free queue ----
    void push_back(int32_t b) {
        Block& x = blocks[b];
        x.prev = tail;
        x.next = -1;
        if (tail >= 0) blocks[tail].next = b; else head = b;
        tail = b;
        x.in_free = true;
        ++nfree;
    }
    void push_front(int32_t b) {
        Block& x = blocks[b];
        x.prev = -1;
        x.next = head;
        if (head >= 0) blocks[head].prev = b; else tail = b;
        head = b;
        x.in_free = true;
        ++nfree;
    }
    void remove(int32_t b) {
        Block& x = blocks[b];
        if (x.prev >= 0) blocks[x.prev].next = x.next; else head = x.next;
        if (x.next >= 0) blocks[x.next].prev = x.prev; else tail = x.prev;
        x.prev = x.next = -1;
        x.in_free = false;
        --nfree;
    }

    void uncache(int32_t b) {
        Block& x = blocks[b];
        if (!x.cached) return;
        auto it = cache.find(x.hash);
        if (it != cache.end() && it->second == b) cache.erase(it);
        x.cached = false;
    }

    // A block from the front of the free queue (its cached hash is evicted).
    int32_t take_free() {
        const int32_t b = head;
        remove(b);
        uncache(b);
        Block& x = blocks[b];
        ++x.gen;
        x.ref = 1;
        return b;
    }

    void release(int32_t b) {
        Block& x = blocks[b];
        if (--x.ref > 0) return;
        if (x.cached) push_back(b);  // keeps its hash; evicted after older ones
        else push_front(b);          // nothing to keep: reused first
    }

    // Register full block i of r (its chain hash is r.chain[i]) if its parent
    // is still the cached holder of r's previous chain hash.
    void register_block(Request& r, size_t i) {
        if (!caching) return;
        const int32_t b = r.table[i];
        int32_t parent = -1;
        if (i > 0) {
            parent = r.table[i - 1];
            const Block& p = blocks[parent];
            if (!p.cached || p.hash != r.chain[i - 1]) return;
        }
        Block& x = blocks[b];
        if (x.cached) return;  // already holds this content (a prefix-cache hit)
        auto it = cache.find(r.chain[i]);
        if (it != cache.end()) uncache(it->second);  // the newest holder wins
        x.cached = true;
        x.hash = r.chain[i];
        x.parent = parent;
        x.parent_gen = parent >= 0 ? blocks[parent].gen : 0;
        x.extra = r.extra;
        memcpy(x.tokens, &r.tokens[i * kBS], sizeof x.tokens);
        cache[x.hash] = b;
    }

    // The cached block holding full block i of a token sequence whose
    // previous block is `parent` (or -1), if any.
    int32_t lookup(uint64_t h, int32_t parent, const int64_t* tokens, uint64_t extra) const {
        auto it = cache.find(h);
        if (it == cache.end()) return -1;
        const Block& x = blocks[it->second];
        if (!x.cached || x.hash != h || x.extra != extra || x.parent != parent) return -1;
        if (parent >= 0 && x.parent_gen != blocks[parent].gen) return -1;
        if (memcmp(x.tokens, tokens, sizeof x.tokens) != 0) return -1;
        return it->second;
    }

    // New blocks (and a copy-on-write block) the next n tokens of r need.
    int32_t blocks_needed(const Request& r, int32_t n) const {
        const int64_t cur = (int64_t)r.tokens.size();
        const int64_t want = (cur + n + kBS - 1) / kBS - (int64_t)r.table.size();
        const bool cow = n > 0 && cur % kBS != 0 && blocks[r.table.back()].ref > 1;
        return (int32_t)(want + (cow ? 1 : 0));
    }
};

namespace {

Request* find(pkv_block_manager* bm, int64_t id) {
    auto it = bm->reqs.find(id);
    return it == bm->reqs.end() ? nullptr : &it->second;
}
const Request* find(const pkv_block_manager* bm, int64_t id) {
    auto it = bm->reqs.find(id);
    return it == bm->reqs.end() ? nullptr : &it->second;
}

}  // namespace

PKV_EXPORT pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t prefix_caching) {
    if (num_blocks < 2) return nullptr;
    pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
    if (bm == nullptr) return nullptr;
    bm->num_blocks = num_blocks;
    bm->caching = prefix_caching != 0;
    bm->blocks.resize((size_t)num_blocks);
    for (int32_t b = 1; b < num_blocks; ++b) bm->push_back(b);  // block 0: the null block
    return bm;
}

PKV_EXPORT void pkv_bm_destroy(pkv_block_manager* bm) { delete bm; }

PKV_EXPORT int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm) {
    return bm == nullptr ? 0 : bm->nfree;
}

PKV_EXPORT int pkv_bm_add_request(pkv_block_manager* bm, int64_t request_id,
                                  const int64_t* prompt_tokens, int32_t num_tokens,
                                  uint64_t extra_key, int32_t* num_cached_tokens) {
    if (bm == nullptr || prompt_tokens == nullptr || num_tokens < 1 ||
        num_cached_tokens == nullptr || bm->reqs.count(request_id) != 0)
        return PKV_ERR_INVALID_ARG;
    Request& r = bm->reqs[request_id];
    r.prompt.assign(prompt_tokens, prompt_tokens + num_tokens);
    r.extra = extra_key;
    int32_t hits = 0;
    if (bm->caching) {
        // full blocks inside the first num_tokens - 1 tokens (the last token
        // is recomputed even on a full hit)
        const int32_t max_hit = (num_tokens - 1) / kBS;
        int32_t parent = -1;
        uint64_t ph = 0;
        for (; hits < max_hit; ++hits) {
            const int64_t* t = prompt_tokens + (size_t)hits * kBS;
            const uint64_t h = block_hash(hits > 0, ph, t, extra_key);
            const int32_t b = bm->lookup(h, parent, t, extra_key);
            if (b < 0) break;
            Block& x = bm->blocks[b];
            if (x.in_free) bm->remove(b);
            ++x.ref;
            r.table.push_back(b);
            r.chain.push_back(h);
            r.tokens.insert(r.tokens.end(), t, t + kBS);
            parent = b;
            ph = h;
        }
        bm->queried += num_tokens;
        bm->hit += (int64_t)hits * kBS;
    }
    *num_cached_tokens = hits * kBS;
    return PKV_OK;
}

PKV_EXPORT int pkv_bm_can_append(const pkv_block_manager* bm, int64_t request_id, int32_t n) {
    if (bm == nullptr || n < 0) return 0;
    const Request* r = find(bm, request_id);
    if (r == nullptr) return 0;
    return bm->blocks_needed(*r, n) <= bm->nfree ? 1 : 0;
}

PKV_EXPORT int pkv_bm_append(pkv_block_manager* bm, int64_t request_id, int32_t n,
                             const int64_t* new_tokens, int64_t* slot_mapping,
                             int32_t copies[][2], int32_t* num_copies) {
    if (bm == nullptr || n < 0 || num_copies == nullptr || (n > 0 && slot_mapping == nullptr) ||
        copies == nullptr)
        return PKV_ERR_INVALID_ARG;
    Request* r = find(bm, request_id);
    if (r == nullptr) return PKV_ERR_INVALID_ARG;
    const int64_t cur = (int64_t)r->tokens.size();
    const int64_t from_prompt = (int64_t)r->prompt.size() > cur ? (int64_t)r->prompt.size() - cur : 0;
    const int64_t generated = n > from_prompt ? n - from_prompt : 0;
    if (generated > 0 && new_tokens == nullptr) return PKV_ERR_INVALID_ARG;
    if (cur + n > INT32_MAX) return PKV_ERR_UNSUPPORTED;
    if (bm->blocks_needed(*r, n) > bm->nfree) return PKV_ERR_WORKSPACE;

    *num_copies = 0;
    if (n > 0 && cur % kBS != 0 && bm->blocks[r->table.back()].ref > 1) {
        // copy-on-write: the shared partial last block is replaced by a copy
        const int32_t src = r->table.back();
        const int32_t dst = bm->take_free();
        --bm->blocks[src].ref;  // still held by the others
        r->table.back() = dst;
        copies[0][0] = src;
        copies[0][1] = dst;
        *num_copies = 1;
    }
    for (int32_t k = 0; k < n; ++k) {
        const int64_t pos = cur + k;
        const int64_t tok = k < from_prompt ? r->prompt[(size_t)pos] : new_tokens[k - from_prompt];
        if (pos % kBS == 0) r->table.push_back(bm->take_free());
        slot_mapping[k] = (int64_t)r->table[(size_t)(pos / kBS)] * kBS + pos % kBS;
        r->tokens.push_back(tok);
        if ((pos + 1) % kBS == 0) {
            // block pos / 16 is full: its chain hash, and the cache entry
            const size_t i = (size_t)(pos / kBS);
            r->chain.push_back(block_hash(i > 0, i > 0 ? r->chain[i - 1] : 0,
                                          &r->tokens[i * kBS], r->extra));
            bm->register_block(*r, i);
        }
    }
    return PKV_OK;
}

PKV_EXPORT int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id) {
    if (bm == nullptr || parent_id == child_id || bm->reqs.count(child_id) != 0)
        return PKV_ERR_INVALID_ARG;
    const Request* p = find(bm, parent_id);
    if (p == nullptr) return PKV_ERR_INVALID_ARG;
    Request copy = *p;
    for (int32_t b : copy.table) ++bm->blocks[b].ref;
    bm->reqs.emplace(child_id, std::move(copy));
    return PKV_OK;
}

PKV_EXPORT int pkv_bm_free_request(pkv_block_manager* bm, int64_t request_id) {
    if (bm == nullptr) return PKV_ERR_INVALID_ARG;
    auto it = bm->reqs.find(request_id);
    if (it == bm->reqs.end()) return PKV_ERR_INVALID_ARG;
    const std::vector<int32_t>& t = it->second.table;
    for (size_t i = t.size(); i-- > 0;) bm->release(t[i]);  // last block first
    bm->reqs.erase(it);
    return PKV_OK;
}

PKV_EXPORT int32_t pkv_bm_num_tokens(const pkv_block_manager* bm, int64_t request_id) {
    if (bm == nullptr) return -1;
    const Request* r = find(bm, request_id);
    return r == nullptr ? -1 : (int32_t)r->tokens.size();
}

PKV_EXPORT int32_t pkv_bm_num_blocks(const pkv_block_manager* bm, int64_t request_id) {
    if (bm == nullptr) return -1;
    const Request* r = find(bm, request_id);
    return r == nullptr ? -1 : (int32_t)r->table.size();
}

PKV_EXPORT int32_t pkv_bm_ref_count(const pkv_block_manager* bm, int32_t block) {
    if (bm == nullptr || block <= 0 || block >= bm->num_blocks) return 0;
    return bm->blocks[(size_t)block].ref;
}

PKV_EXPORT int pkv_bm_block_tables(const pkv_block_manager* bm, const int64_t* request_ids,
                                   int32_t n, int32_t max_blocks, int32_t* block_tables,
                                   int32_t* context_lens) {
    if (bm == nullptr || n < 0 || max_blocks < 1 || (n > 0 && (request_ids == nullptr ||
                                                               block_tables == nullptr)))
        return PKV_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n; ++i) {
        const Request* r = find(bm, request_ids[i]);
        if (r == nullptr) return PKV_ERR_INVALID_ARG;
        if ((int64_t)r->table.size() > max_blocks) return PKV_ERR_UNSUPPORTED;
    }
    for (int32_t i = 0; i < n; ++i) {
        const Request* r = find(bm, request_ids[i]);
        int32_t* row = block_tables + (size_t)i * max_blocks;
        for (int32_t j = 0; j < max_blocks; ++j)
            row[j] = j < (int32_t)r->table.size() ? r->table[(size_t)j] : 0;
        if (context_lens != nullptr) context_lens[i] = (int32_t)r->tokens.size();
    }
    return PKV_OK;
}

PKV_EXPORT int pkv_bm_prefix_groups(const pkv_block_manager* bm, const int64_t* request_ids,
                                    int32_t n, int32_t* group_starts,
                                    int32_t* group_prefix_blocks, int32_t* num_groups) {
    if (bm == nullptr || n < 0 || group_starts == nullptr || group_prefix_blocks == nullptr ||
        num_groups == nullptr || (n > 0 && request_ids == nullptr))
        return PKV_ERR_INVALID_ARG;
    std::vector<const Request*> rs((size_t)n);
    for (int32_t i = 0; i < n; ++i) {
        rs[(size_t)i] = find(bm, request_ids[i]);
        if (rs[(size_t)i] == nullptr) return PKV_ERR_INVALID_ARG;
    }
    auto full_blocks = [](const Request* r) { return (int32_t)(r->tokens.size() / kBS); };
    int32_t ng = 0;
    auto emit = [&](int32_t start, int32_t pre) {
        // consecutive runs without sharing merge into one group
        if (pre == 0 && ng > 0 && group_prefix_blocks[ng - 1] == 0) return;
        group_starts[ng] = start;
        group_prefix_blocks[ng] = pre;
        ++ng;
    };
    int32_t a = 0;
    while (a < n) {
        const Request* lead = rs[(size_t)a];
        int32_t b = a + 1;
        while (b < n && !lead->table.empty() && !rs[(size_t)b]->table.empty() &&
               rs[(size_t)b]->table[0] == lead->table[0])
            ++b;
        int32_t pre = 0;
        if (b - a >= 2) {
            pre = full_blocks(lead);
            for (int32_t m = a + 1; m < b; ++m) {
                const Request* r = rs[(size_t)m];
                int32_t k = 0;
                const int32_t lim = std::min(pre, full_blocks(r));
                while (k < lim && r->table[(size_t)k] == lead->table[(size_t)k]) ++k;
                pre = k;
            }
        }
        emit(a, pre);
        a = b;
    }
    if (n > 0) group_starts[ng] = n;
    else group_starts[0] = 0;
    *num_groups = ng;
    return PKV_OK;
}

PKV_EXPORT void pkv_bm_prefix_cache_stats(const pkv_block_manager* bm, int64_t* queried_tokens,
                                          int64_t* hit_tokens) {
    if (queried_tokens != nullptr) *queried_tokens = bm == nullptr ? 0 : bm->queried;
    if (hit_tokens != nullptr) *hit_tokens = bm == nullptr ? 0 : bm->hit;
}
