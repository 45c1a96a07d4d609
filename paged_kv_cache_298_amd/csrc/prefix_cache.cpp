// prefix_cache.cpp -- host-side prefix cache over the refcounted block allocator.
//
// [P2] "Paged Attention" tutorial (infra.pidoku.co.in), section 5, "The relationship to
// prefix caching": once KV lives in shareable refcounted blocks, a map from the hash of
// a block's token ids to its block id lets a new sequence whose leading blocks hash to
// cached ones point at them (one more reference) instead of computing them again.
//
// Readings taken here:
//   * A block is identified by its own token ids AND everything before it (the K/V of a
//     token depend on the whole prefix), so an entry records its parent entry and the
//     block's tokens, and a lookup walks the chain from the first block. The 64-bit key
//     (splitmix64 over the parent key and the tokens) only finds candidates; a hit needs
//     the parent entry and every token to be equal.
//   * Only full blocks are cached; a sequence's partly filled last block stays private.
//   * Blocks enter the cache when the caller publishes a sequence whose K/V it has
//     written; the cache then holds one reference of its own, so a cached block outlives
//     the sequences that used it.
//   * When a new sequence needs more free blocks than the allocator has, cached blocks
//     that nobody else references are released, least recently used first. An acquire
//     that cannot be satisfied even then fails before anything changes.
//   * Entry ids grow monotonically and are never reused, so an entry whose parent was
//     evicted can no longer match any chain.
#include <stdint.h>
#include <stdio.h>

#include <map>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

struct Entry {
    uint64_t parent;              // 0 for a sequence's first block
    uint64_t key;
    uint64_t stamp;               // last use; the LRU order
    int32_t block;
    std::vector<int32_t> tokens;
};

// splitmix64 finalizer (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", 2014): a cheap 64-bit mix.
uint64_t mix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

uint64_t block_key(uint64_t parent_key, const int32_t* tokens, int32_t n) {
    uint64_t h = mix64(parent_key);
    for (int32_t i = 0; i < n; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i]);
    return h;
}

}  // namespace

struct pa_prefix_cache {
    pa_allocator* alloc;
    int32_t block_size;
    uint64_t next_id = 1;
    uint64_t clock = 0;
    std::unordered_map<uint64_t, Entry> entries;                 // id -> entry
    std::unordered_multimap<uint64_t, uint64_t> by_key;          // key -> id
    std::map<uint64_t, uint64_t> lru;                            // stamp -> id

    // the entry for (parent, tokens), or 0
    uint64_t find(uint64_t parent, uint64_t parent_key, const int32_t* tokens, uint64_t* key) const {
        *key = block_key(parent_key, tokens, block_size);
        auto range = by_key.equal_range(*key);
        for (auto it = range.first; it != range.second; ++it) {
            const Entry& e = entries.at(it->second);
            bool same = e.parent == parent;
            for (int32_t i = 0; same && i < block_size; ++i) same = e.tokens[(size_t)i] == tokens[i];
            if (same) return it->second;
        }
        return 0;
    }
    void touch(uint64_t id) {
        Entry& e = entries.at(id);
        lru.erase(e.stamp);
        e.stamp = ++clock;
        lru.emplace(e.stamp, id);
    }
    void remove(uint64_t id) {
        const Entry& e = entries.at(id);
        auto range = by_key.equal_range(e.key);
        for (auto it = range.first; it != range.second; ++it)
            if (it->second == id) { by_key.erase(it); break; }
        lru.erase(e.stamp);
        entries.erase(id);
    }
    int32_t evictable() const {
        int32_t n = 0;
        for (const auto& kv : entries) n += pa_alloc_refcount(alloc, kv.second.block) == 1;
        return n;
    }
    int32_t evict(int32_t n) {
        int32_t done = 0;
        for (auto it = lru.begin(); it != lru.end() && done < n;) {
            const uint64_t id = it->second;
            ++it;
            const int32_t blk = entries.at(id).block;
            if (pa_alloc_refcount(alloc, blk) != 1) continue;
            remove(id);
            pa_alloc_free(alloc, &blk, 1);
            ++done;
        }
        return done;
    }
};

extern "C" {

pa_prefix_cache* pa_pcache_create(pa_allocator* a) {
    if (!a) {
        pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_pcache_create: null allocator");
        return nullptr;
    }
    pa_prefix_cache* c = new pa_prefix_cache;
    c->alloc = a;
    c->block_size = pa_alloc_block_size(a);
    return c;
}

void pa_pcache_destroy(pa_prefix_cache* c) {
    if (!c) return;
    for (const auto& kv : c->entries) {
        const int32_t blk = kv.second.block;
        pa_alloc_free(c->alloc, &blk, 1);
    }
    delete c;
}

int32_t pa_pcache_acquire(pa_prefix_cache* c, const int32_t* tokens, int32_t n_tokens,
                          int32_t* table, int32_t table_cap, int32_t* n_table,
                          int32_t* n_cached) {
    if (!c || n_tokens < 0 || (n_tokens > 0 && !tokens) || !n_table || !n_cached ||
        table_cap < 0 || (table_cap > 0 && !table))
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_pcache_acquire: bad arguments");
    const int32_t bs = c->block_size;
    const int32_t total = (int32_t)(((int64_t)n_tokens + bs - 1) / bs);
    if (total > table_cap)
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_pcache_acquire: table too small");
    // the longest run of leading full blocks already cached
    std::vector<uint64_t> hits;
    uint64_t parent = 0, parent_key = 0;
    for (int32_t i = 0; i < n_tokens / bs; ++i) {
        uint64_t key;
        const uint64_t id = c->find(parent, parent_key, tokens + (int64_t)i * bs, &key);
        if (!id) break;
        hits.push_back(id);
        parent = id;
        parent_key = key;
    }
    const int32_t nh = (int32_t)hits.size();
    const int32_t need = total - nh;
    // feasibility before any change: free blocks plus cached blocks nobody else holds,
    // other than the hits themselves
    int32_t spare = pa_alloc_num_free(c->alloc);
    if (spare < need) {
        int32_t ev = c->evictable();
        for (uint64_t id : hits) ev -= pa_alloc_refcount(c->alloc, c->entries.at(id).block) == 1;
        if (spare + ev < need) {
            char buf[96];
            snprintf(buf, sizeof buf, "out of KV blocks: need %d, have %d", need, spare + ev);
            return pa_internal::set_error(PA_ERR_NO_BLOCKS, buf);
        }
    }
    for (int32_t i = 0; i < nh; ++i) table[i] = c->entries.at(hits[(size_t)i]).block;
    if (nh > 0 && pa_alloc_fork(c->alloc, table, nh, table) != PA_OK) return PA_ERR_INVALID_ARG;
    if (spare < need) c->evict(need - spare);   // the hits now hold two references
    if (need > 0 && pa_alloc_allocate(c->alloc, need, table + nh) != PA_OK) {
        pa_alloc_free(c->alloc, table, nh);
        return PA_ERR_NO_BLOCKS;
    }
    for (uint64_t id : hits) c->touch(id);
    *n_table = total;
    *n_cached = nh * bs;
    return PA_OK;
}

int32_t pa_pcache_publish(pa_prefix_cache* c, const int32_t* tokens, int32_t n_tokens,
                          const int32_t* table, int32_t n_table) {
    if (!c || n_tokens < 0 || (n_tokens > 0 && !tokens) || n_table < 0 || (n_table > 0 && !table))
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_pcache_publish: bad arguments");
    const int32_t bs = c->block_size;
    const int32_t full = n_tokens / bs;
    if (full > n_table)
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_pcache_publish: table shorter than the tokens");
    for (int32_t i = 0; i < full; ++i)
        if (pa_alloc_refcount(c->alloc, table[i]) < 1)
            return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_pcache_publish: a table block is not allocated");
    uint64_t parent = 0, parent_key = 0;
    for (int32_t i = 0; i < full; ++i) {
        uint64_t key;
        uint64_t id = c->find(parent, parent_key, tokens + (int64_t)i * bs, &key);
        if (!id) {
            id = c->next_id++;
            Entry e;
            e.parent = parent;
            e.key = key;
            e.stamp = 0;
            e.block = table[i];
            e.tokens.assign(tokens + (int64_t)i * bs, tokens + (int64_t)(i + 1) * bs);
            const int32_t blk = table[i];
            pa_alloc_fork(c->alloc, &blk, 1, &e.block);   // the cache's own reference
            c->entries.emplace(id, std::move(e));
            c->by_key.emplace(key, id);
        }
        c->touch(id);
        parent = id;
        parent_key = key;
    }
    return PA_OK;
}

int32_t pa_pcache_evict(pa_prefix_cache* c, int32_t n) {
    if (!c || n < 0) return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_pcache_evict: bad arguments");
    return c->evict(n);
}

int32_t pa_pcache_num_entries(const pa_prefix_cache* c) {
    return c ? (int32_t)c->entries.size() : 0;
}

}  // extern "C"
