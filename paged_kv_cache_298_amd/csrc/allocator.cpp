// allocator.cpp -- host-side refcounted pool of physical KV block ids that builds block
// tables.
//
// Behaviour ([P2] "Paged Attention" tutorial, infra.pidoku.co.in, section 4 "Tiny
// example" and section 5 "Copy-on-write sharing"; [P4] "PagedAttention & KV-Cache
// Management in High-Throughput LLM Serving", subroutine-cs.cc, section 3):
//   - free ids are handed out last in, first out; a new pool has id 0 on top and
//     id num_blocks-1 at the bottom (or the caller's order);
//   - a request for n ids is met whole or not at all: the n topmost ids, listed from the
//     deepest of them to the top one, each with one holder;
//   - releasing an id drops one holder; with none left it goes back on top;
//   - sharing (fork) adds one holder per id;
//   - a token written into a block other sequences still hold goes to a fresh private
//     block, after a copy of the shared one when it already holds tokens of the sequence.
// Every failing call leaves the pool and the caller's table unchanged.
//
// Layout: the free ids form a stack threaded through one array (under[b] = the free id
// directly below b, -1 at the bottom), so taking, returning and counting are O(1) per id
// and need no allocation after creation.
#include <stdio.h>

#include <algorithm>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

struct pa_allocator {
    int32_t num_blocks;
    int32_t block_size;
    std::vector<int32_t> holders;   // per id; 0 = free
    std::vector<int32_t> under;     // per free id: the free id below it, -1 at the bottom
    int32_t top;                    // topmost free id, -1 when none is free
    int32_t n_free;

    void push(int32_t b) {
        under[(size_t)b] = top;
        top = b;
        ++n_free;
    }
    int32_t pop() {
        const int32_t b = top;
        top = under[(size_t)b];
        --n_free;
        return b;
    }
    bool valid(int32_t b) const { return b >= 0 && b < num_blocks; }
    bool held(int32_t b) const { return valid(b) && holders[(size_t)b] > 0; }
};

namespace {

int32_t bad(const char* msg) { return pa_internal::set_error(PA_ERR_INVALID_ARG, msg); }

int32_t no_blocks(int32_t need, int32_t have) {
    char buf[96];
    snprintf(buf, sizeof buf, "out of KV blocks: need %d, have %d", need, have);
    return pa_internal::set_error(PA_ERR_NO_BLOCKS, buf);
}

// a fresh private block: the top free id, with one holder (caller checked n_free > 0)
int32_t take_one(pa_allocator* a) {
    const int32_t b = a->pop();
    a->holders[(size_t)b] = 1;
    return b;
}

}  // namespace

extern "C" {

pa_allocator* pa_alloc_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* initial_free_order) {
    if (num_blocks < 0 || block_size <= 0) {
        bad("pa_alloc_create: num_blocks must be >= 0 and block_size > 0");
        return nullptr;
    }
    if (initial_free_order) {
        std::vector<int32_t> ids(initial_free_order, initial_free_order + num_blocks);
        std::sort(ids.begin(), ids.end());
        for (int32_t i = 0; i < num_blocks; ++i) {
            if (ids[(size_t)i] != i) {
                bad("pa_alloc_create: initial_free_order must list each block id once");
                return nullptr;
            }
        }
    }
    pa_allocator* a = new pa_allocator;
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->holders.assign((size_t)num_blocks, 0);
    a->under.assign((size_t)num_blocks, -1);
    a->top = -1;
    a->n_free = 0;
    // bottom first: the caller's order, else num_blocks-1 down to 0
    for (int32_t i = 0; i < num_blocks; ++i)
        a->push(initial_free_order ? initial_free_order[i] : num_blocks - 1 - i);
    pa_internal::clear_error();
    return a;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int32_t pa_alloc_allocate(pa_allocator* a, int32_t n, int32_t* out) {
    if (!a || n < 0 || (n > 0 && !out)) return bad("pa_alloc_allocate: bad arguments");
    if (n > a->n_free) return no_blocks(n, a->n_free);
    // the top id is the last of the n listed
    for (int32_t i = n - 1; i >= 0; --i) out[i] = take_one(a);
    return pa_internal::clear_error();
}

int32_t pa_alloc_free(pa_allocator* a, const int32_t* blocks, int32_t n) {
    if (!a || n < 0 || (n > 0 && !blocks)) return bad("pa_alloc_free: bad arguments");
    // check the whole list first (an id listed k times needs k holders)
    std::vector<int32_t> ids(blocks, blocks + n);
    std::sort(ids.begin(), ids.end());
    for (size_t i = 0; i < ids.size();) {
        size_t j = i;
        while (j < ids.size() && ids[j] == ids[i]) ++j;
        if (!a->valid(ids[i])) return bad("pa_alloc_free: block id out of range");
        if ((int64_t)(j - i) > a->holders[(size_t)ids[i]])
            return bad("pa_alloc_free: block freed more often than it is referenced");
        i = j;
    }
    for (int32_t i = 0; i < n; ++i)
        if (--a->holders[(size_t)blocks[i]] == 0) a->push(blocks[i]);
    return pa_internal::clear_error();
}

int32_t pa_alloc_fork(pa_allocator* a, const int32_t* blocks, int32_t n, int32_t* out) {
    if (!a || n < 0 || (n > 0 && (!blocks || !out))) return bad("pa_alloc_fork: bad arguments");
    for (int32_t i = 0; i < n; ++i)
        if (!a->held(blocks[i])) return bad("pa_alloc_fork: block is not allocated");
    for (int32_t i = 0; i < n; ++i) {
        ++a->holders[(size_t)blocks[i]];
        out[i] = blocks[i];
    }
    return pa_internal::clear_error();
}

int32_t pa_alloc_append_token(pa_allocator* a, int32_t* table, int32_t* n_table,
                              int32_t table_cap, int32_t* seq_len, int32_t* out_slot,
                              int32_t* out_cow_src, int32_t* out_cow_dst) {
    if (!a || !table || !n_table || !seq_len || !out_slot || !out_cow_src || !out_cow_dst)
        return bad("pa_alloc_append_token: null argument");
    const int32_t bs = a->block_size;
    const int32_t pos = *seq_len;
    const int32_t used = *n_table;
    if (pos < 0 || used < 0 || used > table_cap) return bad("pa_alloc_append_token: bad sequence state");
    const int32_t blk = pos / bs;
    const int32_t off = pos % bs;
    if (blk > used) return bad("pa_alloc_append_token: block table shorter than the sequence");
    const bool grows = blk == used;
    if (grows && used == table_cap) return bad("pa_alloc_append_token: block table is full");
    if (!grows && !a->held(table[blk]))
        return bad("pa_alloc_append_token: table names a block that is not allocated");
    const bool shared = !grows && a->holders[(size_t)table[blk]] > 1;
    if ((grows || shared) && a->n_free == 0) return no_blocks(1, 0);

    int32_t src = -1, dst = -1;
    if (grows) {
        table[used] = take_one(a);
        *n_table = used + 1;
    } else if (shared) {
        const int32_t old = table[blk];
        table[blk] = take_one(a);
        --a->holders[(size_t)old];
        if (off != 0) {   // the shared block already holds earlier tokens of this sequence
            src = old;
            dst = table[blk];
        }
    }
    *out_slot = table[blk] * bs + off;
    *out_cow_src = src;
    *out_cow_dst = dst;
    *seq_len = pos + 1;
    return pa_internal::clear_error();
}

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
    if (!a || !a->valid(block)) return bad("pa_alloc_refcount: block id out of range");
    return a->holders[(size_t)block];
}

int32_t pa_alloc_block_size(const pa_allocator* a) { return a ? a->block_size : 0; }

int32_t pa_alloc_num_free(const pa_allocator* a) {
    if (!a) return bad("pa_alloc_num_free: null allocator");
    return a->n_free;
}

int32_t pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap) {
    if (!a || cap < 0 || (cap > 0 && !out)) return bad("pa_alloc_free_list: bad arguments");
    // walk from the top down, then report bottom to top
    std::vector<int32_t> down;
    down.reserve((size_t)a->n_free);
    for (int32_t b = a->top; b >= 0; b = a->under[(size_t)b]) down.push_back(b);
    const int32_t n = (int32_t)down.size();
    for (int32_t i = 0; i < n && i < cap; ++i) out[i] = down[(size_t)(n - 1 - i)];
    return n;
}

}  // extern "C"
