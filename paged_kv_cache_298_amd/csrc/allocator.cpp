// allocator.cpp -- host-side refcounted block allocator that builds block tables.
//
// Follows the block manager of [P2] "Paged Attention" tutorial (infra.pidoku.co.in),
// section 4 "Tiny example": a stack of free physical block ids (initially N-1 ... 0, top
// at the end), all-or-nothing allocation of the top n ids in stack order, a refcount per
// block, free = decrement and push back at zero, fork = increment. The append path adds
// the copy-on-write rule of section 5 "Copy-on-write sharing" and of [P4]
// "PagedAttention & KV-Cache Management in High-Throughput LLM Serving"
// (subroutine-cs.cc), section 3: a token that would land in a block other sequences still
// reference goes to a fresh block instead, after a copy of the old one when it already
// holds tokens of this sequence. Unlike the page's Go code, every failure leaves the
// allocator and the sequence unchanged (the page bumps the length before allocating).
#include <stdio.h>

#include <unordered_map>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

struct pa_allocator {
    int32_t num_blocks;
    int32_t block_size;
    std::vector<int32_t> free_stack;    // bottom ... top
    std::vector<int32_t> refcount;      // per block id; 0 = free
};

namespace {

int32_t bad(const char* msg) { return pa_internal::set_error(PA_ERR_INVALID_ARG, msg); }

int32_t no_blocks(int32_t need, int32_t have) {
    char buf[96];
    snprintf(buf, sizeof buf, "out of KV blocks: need %d, have %d", need, have);
    return pa_internal::set_error(PA_ERR_NO_BLOCKS, buf);
}

bool in_range(const pa_allocator* a, int32_t b) { return b >= 0 && b < a->num_blocks; }

}  // namespace

extern "C" {

pa_allocator* pa_alloc_create(int32_t num_blocks, int32_t block_size,
                              const int32_t* initial_free_order) {
    if (num_blocks < 0 || block_size <= 0) {
        bad("pa_alloc_create: num_blocks must be >= 0 and block_size > 0");
        return nullptr;
    }
    pa_allocator* a = new pa_allocator;
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->refcount.assign((size_t)num_blocks, 0);
    a->free_stack.reserve((size_t)num_blocks);
    if (initial_free_order) {
        std::vector<char> seen((size_t)num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            const int32_t b = initial_free_order[i];
            if (!in_range(a, b) || seen[(size_t)b]) {
                delete a;
                bad("pa_alloc_create: initial_free_order must list each block id once");
                return nullptr;
            }
            seen[(size_t)b] = 1;
            a->free_stack.push_back(b);
        }
    } else {
        for (int32_t b = num_blocks - 1; b >= 0; --b) a->free_stack.push_back(b);
    }
    pa_internal::clear_error();
    return a;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int32_t pa_alloc_allocate(pa_allocator* a, int32_t n, int32_t* out) {
    if (!a || n < 0 || (n > 0 && !out)) return bad("pa_alloc_allocate: bad arguments");
    const int32_t have = (int32_t)a->free_stack.size();
    if (n > have) return no_blocks(n, have);
    const size_t cut = a->free_stack.size() - (size_t)n;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t b = a->free_stack[cut + (size_t)i];
        out[i] = b;
        a->refcount[(size_t)b] = 1;
    }
    a->free_stack.resize(cut);
    return pa_internal::clear_error();
}

int32_t pa_alloc_free(pa_allocator* a, const int32_t* blocks, int32_t n) {
    if (!a || n < 0 || (n > 0 && !blocks)) return bad("pa_alloc_free: bad arguments");
    // check first, so that a bad list changes nothing
    std::unordered_map<int32_t, int32_t> uses;
    for (int32_t i = 0; i < n; ++i) {
        if (!in_range(a, blocks[i])) return bad("pa_alloc_free: block id out of range");
        const int32_t k = ++uses[blocks[i]];
        if (k > a->refcount[(size_t)blocks[i]])
            return bad("pa_alloc_free: block freed more often than it is referenced");
    }
    for (int32_t i = 0; i < n; ++i) {
        int32_t& rc = a->refcount[(size_t)blocks[i]];
        if (--rc == 0) a->free_stack.push_back(blocks[i]);
    }
    return pa_internal::clear_error();
}

int32_t pa_alloc_fork(pa_allocator* a, const int32_t* blocks, int32_t n, int32_t* out) {
    if (!a || n < 0 || (n > 0 && (!blocks || !out))) return bad("pa_alloc_fork: bad arguments");
    for (int32_t i = 0; i < n; ++i) {
        if (!in_range(a, blocks[i]) || a->refcount[(size_t)blocks[i]] <= 0)
            return bad("pa_alloc_fork: block is not allocated");
    }
    for (int32_t i = 0; i < n; ++i) {
        ++a->refcount[(size_t)blocks[i]];
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
    const int32_t n = *n_table;
    if (pos < 0 || n < 0 || n > table_cap) return bad("pa_alloc_append_token: bad sequence state");
    const int32_t j = pos / bs;
    int32_t src = -1, dst = -1;
    if (j > n) return bad("pa_alloc_append_token: block table shorter than the sequence");
    if (j == n) {
        if (n == table_cap) return bad("pa_alloc_append_token: block table is full");
        if (a->free_stack.empty()) return no_blocks(1, 0);
        const int32_t fresh = a->free_stack.back();
        a->free_stack.pop_back();
        a->refcount[(size_t)fresh] = 1;
        table[n] = fresh;
        *n_table = n + 1;
    } else {
        const int32_t cur = table[j];
        if (!in_range(a, cur) || a->refcount[(size_t)cur] <= 0)
            return bad("pa_alloc_append_token: table names a block that is not allocated");
        if (a->refcount[(size_t)cur] > 1) {
            if (a->free_stack.empty()) return no_blocks(1, 0);
            const int32_t fresh = a->free_stack.back();
            a->free_stack.pop_back();
            a->refcount[(size_t)fresh] = 1;
            --a->refcount[(size_t)cur];
            table[j] = fresh;
            if (pos % bs != 0) {
                src = cur;
                dst = fresh;
            }
        }
    }
    *out_slot = table[j] * bs + pos % bs;
    *out_cow_src = src;
    *out_cow_dst = dst;
    *seq_len = pos + 1;
    return pa_internal::clear_error();
}

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
    if (!a || !in_range(a, block)) return bad("pa_alloc_refcount: block id out of range");
    return a->refcount[(size_t)block];
}

int32_t pa_alloc_block_size(const pa_allocator* a) { return a ? a->block_size : 0; }

int32_t pa_alloc_num_free(const pa_allocator* a) {
    if (!a) return bad("pa_alloc_num_free: null allocator");
    return (int32_t)a->free_stack.size();
}

int32_t pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap) {
    if (!a || cap < 0 || (cap > 0 && !out)) return bad("pa_alloc_free_list: bad arguments");
    const int32_t n = (int32_t)a->free_stack.size();
    for (int32_t i = 0; i < n && i < cap; ++i) out[i] = a->free_stack[(size_t)i];
    return n;
}

}  // extern "C"
