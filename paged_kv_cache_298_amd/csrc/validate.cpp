// validate.cpp -- the debug validation pass: checks of the device-resident preconditions
// that the kernels assume and do not check (they clamp what they read so that a violation
// never reaches outside the buffers, but its rows come out wrong and nothing reports it).
//
// The preconditions come from the pages' model of the cache:
//   - a sequence's table names a physical block for each of its ceil(L / block_size)
//     logical blocks ([P1] "PagedAttention", "Interpret Block Tables"; [P2] "Paged
//     Attention", section 4 "Tiny example", PhysicalIndex);
//   - each new token has its own slot, so no two tokens write the same cache row;
//   - a copy-on-write clone goes to a fresh block that is then written ([P2] section 5
//     "Copy-on-write sharing": copy first, then write), so the destinations are distinct
//     and none of them is a block another pair copies from.
// The host validators (pa_validate_*) read host copies. pa_set_validation(1), or the
// environment variable PA_VALIDATE=1 when the library loads, makes every kernel entry
// point copy its index arrays to the host on its stream, wait, validate them and return
// PA_ERR_INVALID_ARG, with nothing enqueued, when one is broken.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace {

int32_t g_validate = -1;   // -1: not read from the environment yet
std::mutex g_validate_mu;

// First violation found: its flag, message and the running flag set.
struct Findings {
    uint32_t flags = 0;
    std::string first;
    void add(uint32_t flag, const char* fmt, ...) {
        if (first.empty()) {
            char buf[256];
            va_list ap;
            va_start(ap, fmt);
            vsnprintf(buf, sizeof buf, fmt, ap);
            va_end(ap);
            first = buf;
        }
        flags |= flag;
    }
    int32_t finish(const char* who, uint32_t* out_flags) {
        if (out_flags) *out_flags = flags;
        if (flags == 0) return pa_internal::clear_error();
        const std::string msg = std::string(who) + ": " + first;
        return pa_internal::set_error(PA_ERR_INVALID_ARG, msg.c_str());
    }
};

void check_tables(Findings& f, const int32_t* tables, const int32_t* lens, int32_t B,
                  int32_t block_size, int32_t num_blocks, int32_t max_blocks) {
    const int64_t cap = (int64_t)block_size * max_blocks;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t L = lens[b];
        if (L < 0 || L > cap) {
            f.add(PA_BAD_LENGTH, "seq_lens[%d] = %d outside [0, %lld]", b, L, (long long)cap);
            continue;
        }
        const int32_t n = (int32_t)((L + block_size - 1) / block_size);
        for (int32_t j = 0; j < n; ++j) {
            const int32_t e = tables[(int64_t)b * max_blocks + j];
            if (e < 0 || e >= num_blocks)
                f.add(PA_BAD_TABLE_ENTRY, "block_tables[%d][%d] = %d outside [0, %d)", b, j, e, num_blocks);
        }
    }
}

void check_slots(Findings& f, const int32_t* slots, int32_t T, int32_t block_size, int32_t num_blocks) {
    const int64_t nslots = (int64_t)block_size * num_blocks;
    std::vector<std::pair<int32_t, int32_t>> used;   // (slot, token)
    used.reserve((size_t)T);
    for (int32_t i = 0; i < T; ++i) {
        const int32_t s = slots[i];
        if (s < 0) continue;   // padding
        if (s >= nslots) {
            f.add(PA_BAD_SLOT, "slot_mapping[%d] = %d outside [0, %lld)", i, s, (long long)nslots);
            continue;
        }
        used.emplace_back(s, i);
    }
    std::sort(used.begin(), used.end());
    for (size_t k = 1; k < used.size(); ++k)
        if (used[k].first == used[k - 1].first)
            f.add(PA_DUP_SLOT, "slot_mapping[%d] and slot_mapping[%d] both name slot %d",
                  used[k - 1].second, used[k].second, used[k].first);
}

// pa_decode_append: a given slot must be where position L - 1 of its sequence lives
void check_append(Findings& f, const int32_t* slots, const int32_t* tables, const int32_t* lens, int32_t B,
                  int32_t block_size, int32_t max_blocks) {
    const int64_t cap = (int64_t)block_size * max_blocks;
    for (int32_t b = 0; b < B; ++b) {
        const int32_t s = slots[b];
        if (s < 0) continue;
        const int32_t L = lens[b];
        if (L < 1 || L > cap) {
            f.add(PA_BAD_APPEND_SLOT, "slot_mapping[%d] = %d given for a sequence of %d tokens", b, s, L);
            continue;
        }
        const int32_t pos = L - 1;
        const int64_t want = (int64_t)tables[(int64_t)b * max_blocks + pos / block_size] * block_size + pos % block_size;
        if (s != want)
            f.add(PA_BAD_APPEND_SLOT, "slot_mapping[%d] = %d, but position %d of sequence %d lives in slot %lld",
                  b, s, pos, b, (long long)want);
    }
}

void check_pairs(Findings& f, const int32_t* pairs, int32_t N, int32_t num_blocks) {
    std::vector<std::pair<int32_t, int32_t>> dst;   // (destination, pair)
    std::vector<int32_t> src;
    for (int32_t i = 0; i < N; ++i) {
        const int32_t s = pairs[2 * (int64_t)i], d = pairs[2 * (int64_t)i + 1];
        if (s < 0 || s >= num_blocks || d < 0 || d >= num_blocks) {
            f.add(PA_BAD_PAIR, "block_pairs[%d] = (%d, %d) outside [0, %d)", i, s, d, num_blocks);
            continue;
        }
        dst.emplace_back(d, i);
        src.push_back(s);
    }
    std::sort(dst.begin(), dst.end());
    std::sort(src.begin(), src.end());
    for (size_t k = 1; k < dst.size(); ++k)
        if (dst[k].first == dst[k - 1].first)
            f.add(PA_DUP_DST, "block_pairs[%d] and block_pairs[%d] both copy into block %d",
                  dst[k - 1].second, dst[k].second, dst[k].first);
    for (const auto& d : dst)
        if (std::binary_search(src.begin(), src.end(), d.first))
            f.add(PA_DST_IS_SRC, "block %d (block_pairs[%d]) is copied into and also copied from",
                  d.first, d.second);
}

void check_groups(Findings& f, const int32_t* groups, int32_t n_groups, const int32_t* tables,
                  const int32_t* lens, int32_t B, int32_t block_size, int32_t max_blocks,
                  int32_t max_members, int32_t max_shared_tokens) {
    int32_t next_free = 0;   // groups are sorted by first sequence and disjoint
    for (int32_t i = 0; i < n_groups; ++i) {
        const int32_t first = groups[3 * (int64_t)i], members = groups[3 * (int64_t)i + 1],
                      shared = groups[3 * (int64_t)i + 2];
        if (first < next_free || members < 1 || members > max_members || first > B - members ||
            shared < 0 || shared > max_shared_tokens) {
            f.add(PA_BAD_GROUP, "groups[%d] = (%d, %d, %d) breaks the order, member or token bounds",
                  i, first, members, shared);
            continue;
        }
        next_free = first + members;
        const int32_t nblk = (shared + block_size - 1) / block_size;
        for (int32_t m = 0; m < members; ++m) {
            const int32_t b = first + m;
            if (lens[b] < shared) {
                f.add(PA_BAD_GROUP, "groups[%d]: seq_lens[%d] = %d is shorter than its %d shared tokens",
                      i, b, lens[b], shared);
                continue;
            }
            for (int32_t j = 0; j < nblk && j < max_blocks; ++j)
                if (tables[(int64_t)b * max_blocks + j] != tables[(int64_t)first * max_blocks + j]) {
                    f.add(PA_BAD_GROUP, "groups[%d]: block_tables[%d][%d] differs from the first member's",
                          i, b, j);
                    break;
                }
        }
    }
}

void check_query_starts(Findings& f, const int32_t* q_starts, const int32_t* lens, int32_t B,
                        int32_t total_q, int32_t max_q) {
    if (q_starts[0] != 0 || q_starts[B] != total_q)
        f.add(PA_BAD_QUERY_STARTS, "q_starts[0] = %d and q_starts[%d] = %d (want 0 and %d)",
              q_starts[0], B, q_starts[B], total_q);
    for (int32_t b = 0; b < B; ++b) {
        const int32_t n = q_starts[b + 1] - q_starts[b];
        const int32_t L = lens[b] < 0 ? 0 : lens[b];
        if (n < 0 || n > max_q || n > L)
            f.add(PA_BAD_QUERY_STARTS, "sequence %d has %d queries (allowed 0 .. min(%d, max_q %d))",
                  b, n, L, max_q);
    }
}

// device -> host copy of n int32 values on the call's stream (waits for it)
int32_t fetch(std::vector<int32_t>& dst, const int32_t* src, int64_t n, void* stream, const char* who) {
    dst.assign((size_t)(n > 0 ? n : 0), 0);
    if (n <= 0) return PA_OK;
    const char* err = "";
    if (pa_internal::copy_to_host(dst.data(), src, (size_t)n * sizeof(int32_t), stream, &err) != 0) {
        const std::string msg = std::string(who) + ": validation copy failed: " + err;
        return pa_internal::set_error(PA_ERR_HIP, msg.c_str());
    }
    return PA_OK;
}

}  // namespace

namespace pa_internal {

bool validation_on() {
    std::lock_guard<std::mutex> lock(g_validate_mu);
    if (g_validate < 0) {
        const char* e = getenv("PA_VALIDATE");
        g_validate = (e && e[0] && e[0] != '0') ? 1 : 0;
    }
    return g_validate == 1;
}

int32_t validate_decode_device(const char* who, const int32_t* tables, const int32_t* lens, int32_t B,
                               int32_t block_size, int32_t num_blocks, int32_t max_blocks, void* stream) {
    std::vector<int32_t> t, l;
    int32_t st = fetch(l, lens, B, stream, who);
    if (st == PA_OK) st = fetch(t, tables, (int64_t)B * max_blocks, stream, who);
    if (st != PA_OK) return st;
    Findings f;
    check_tables(f, t.data(), l.data(), B, block_size, num_blocks, max_blocks);
    return f.finish(who, nullptr);
}

int32_t validate_shared_device(const int32_t* tables, const int32_t* lens, const int32_t* groups,
                               int32_t n_groups, int32_t B, int32_t block_size, int32_t num_blocks,
                               int32_t max_blocks, int32_t max_members, int32_t max_shared_tokens,
                               void* stream) {
    const char* who = "pa_decode_shared";
    std::vector<int32_t> t, l, g;
    int32_t st = fetch(l, lens, B, stream, who);
    if (st == PA_OK) st = fetch(t, tables, (int64_t)B * max_blocks, stream, who);
    if (st == PA_OK) st = fetch(g, groups, (int64_t)n_groups * 3, stream, who);
    if (st != PA_OK) return st;
    Findings f;
    check_tables(f, t.data(), l.data(), B, block_size, num_blocks, max_blocks);
    if (f.flags == 0)
        check_groups(f, g.data(), n_groups, t.data(), l.data(), B, block_size, max_blocks, max_members,
                     max_shared_tokens);
    return f.finish(who, nullptr);
}

int32_t validate_multi_device(const int32_t* tables, const int32_t* lens, const int32_t* q_starts,
                              int32_t B, int32_t total_q, int32_t max_q, int32_t block_size,
                              int32_t num_blocks, int32_t max_blocks, void* stream) {
    const char* who = "pa_decode_multi";
    std::vector<int32_t> t, l, qs;
    int32_t st = fetch(l, lens, B, stream, who);
    if (st == PA_OK) st = fetch(t, tables, (int64_t)B * max_blocks, stream, who);
    if (st == PA_OK) st = fetch(qs, q_starts, (int64_t)B + 1, stream, who);
    if (st != PA_OK) return st;
    Findings f;
    check_tables(f, t.data(), l.data(), B, block_size, num_blocks, max_blocks);
    check_query_starts(f, qs.data(), l.data(), B, total_q, max_q);
    return f.finish(who, nullptr);
}

int32_t validate_slots_device(const int32_t* slots, int32_t T, int32_t block_size, int32_t num_blocks,
                              void* stream) {
    const char* who = "pa_reshape_and_cache";
    std::vector<int32_t> s;
    const int32_t st = fetch(s, slots, T, stream, who);
    if (st != PA_OK) return st;
    Findings f;
    check_slots(f, s.data(), T, block_size, num_blocks);
    return f.finish(who, nullptr);
}

int32_t validate_append_device(const int32_t* slots, const int32_t* tables, const int32_t* lens, int32_t B,
                               int32_t block_size, int32_t num_blocks, int32_t max_blocks, void* stream) {
    const char* who = "pa_decode_append";
    std::vector<int32_t> s, t, l;
    int32_t st = fetch(s, slots, B, stream, who);
    if (st == PA_OK) st = fetch(l, lens, B, stream, who);
    if (st == PA_OK) st = fetch(t, tables, (int64_t)B * max_blocks, stream, who);
    if (st != PA_OK) return st;
    Findings f;
    check_slots(f, s.data(), B, block_size, num_blocks);
    check_append(f, s.data(), t.data(), l.data(), B, block_size, max_blocks);
    return f.finish(who, nullptr);
}

int32_t validate_pairs_device(const int32_t* pairs, int32_t N, int32_t num_blocks, void* stream) {
    const char* who = "pa_copy_blocks";
    std::vector<int32_t> p;
    const int32_t st = fetch(p, pairs, (int64_t)N * 2, stream, who);
    if (st != PA_OK) return st;
    Findings f;
    check_pairs(f, p.data(), N, num_blocks);
    return f.finish(who, nullptr);
}

}  // namespace pa_internal

extern "C" {

int32_t pa_set_validation(int32_t on) {
    if (on != 0 && on != 1)
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_set_validation: on must be 0 or 1");
    std::lock_guard<std::mutex> lock(g_validate_mu);
    g_validate = on;
    return pa_internal::clear_error();
}

int32_t pa_validation_enabled(void) { return pa_internal::validation_on() ? 1 : 0; }

int32_t pa_validate_decode(const int32_t* block_tables, const int32_t* seq_lens, int32_t B,
                           int32_t block_size, int32_t num_blocks, int32_t max_blocks,
                           uint32_t* flags) {
    if (B < 0 || block_size <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
        (B > 0 && (!block_tables || !seq_lens)))
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_validate_decode: bad arguments");
    Findings f;
    check_tables(f, block_tables, seq_lens, B, block_size, num_blocks, max_blocks);
    return f.finish("pa_validate_decode", flags);
}

int32_t pa_validate_slots(const int32_t* slot_mapping, int32_t T, int32_t block_size,
                          int32_t num_blocks, uint32_t* flags) {
    if (T < 0 || block_size <= 0 || num_blocks <= 0 || (T > 0 && !slot_mapping))
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_validate_slots: bad arguments");
    Findings f;
    check_slots(f, slot_mapping, T, block_size, num_blocks);
    return f.finish("pa_validate_slots", flags);
}

int32_t pa_validate_append(const int32_t* slot_mapping, const int32_t* block_tables,
                           const int32_t* seq_lens, int32_t B, int32_t block_size, int32_t num_blocks,
                           int32_t max_blocks, uint32_t* flags) {
    if (B < 0 || block_size <= 0 || num_blocks <= 0 || max_blocks <= 0 ||
        (B > 0 && (!slot_mapping || !block_tables || !seq_lens)))
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_validate_append: bad arguments");
    Findings f;
    check_slots(f, slot_mapping, B, block_size, num_blocks);
    check_append(f, slot_mapping, block_tables, seq_lens, B, block_size, max_blocks);
    return f.finish("pa_validate_append", flags);
}

int32_t pa_validate_block_pairs(const int32_t* block_pairs, int32_t N, int32_t num_blocks,
                                uint32_t* flags) {
    if (N < 0 || num_blocks <= 0 || (N > 0 && !block_pairs))
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_validate_block_pairs: bad arguments");
    Findings f;
    check_pairs(f, block_pairs, N, num_blocks);
    return f.finish("pa_validate_block_pairs", flags);
}

int32_t pa_validate_groups(const int32_t* groups, int32_t n_groups, const int32_t* block_tables,
                           const int32_t* seq_lens, int32_t B, int32_t block_size,
                           int32_t max_blocks, int32_t max_members, int32_t max_shared_tokens,
                           uint32_t* flags) {
    if (n_groups < 0 || B < 0 || block_size <= 0 || max_blocks <= 0 ||
        (n_groups > 0 && (!groups || !block_tables || !seq_lens)))
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_validate_groups: bad arguments");
    Findings f;
    check_groups(f, groups, n_groups, block_tables, seq_lens, B, block_size, max_blocks, max_members,
                 max_shared_tokens);
    return f.finish("pa_validate_groups", flags);
}

int32_t pa_validate_query_starts(const int32_t* q_starts, const int32_t* seq_lens, int32_t B,
                                 int32_t total_q, int32_t max_q, uint32_t* flags) {
    if (B < 0 || total_q < 0 || max_q < 0 || !q_starts || (B > 0 && !seq_lens))
        return pa_internal::set_error(PA_ERR_INVALID_ARG, "pa_validate_query_starts: bad arguments");
    Findings f;
    check_query_starts(f, q_starts, seq_lens, B, total_q, max_q);
    return f.finish("pa_validate_query_starts", flags);
}

}  // extern "C"
