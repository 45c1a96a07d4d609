// pa_multi.hip -- the shared-prefix and multi-query attention kernels for gfx950.
//
// Shared prefix ([P1] "PagedAttention" on shared prompts and parallel sampling; [P2]
// "Paged Attention" tutorial, section 5 "Copy-on-write sharing"): the leading blocks a
// group of sequences shares are read once for all of them (decode_shared_kernel), then
// each member's own tokens; decode_reduce_kernel merges the partial states.
// Multi-query ([P4] "PagedAttention & KV-Cache Management in High-Throughput LLM
// Serving", section 1: the prefill phase computes all prompt tokens in parallel): several
// of a sequence's newest tokens attend at once under a causal mask (decode_multi_kernel).
// Both put the query rows (members x heads, or tokens x heads) in the columns of the
// score tiles, so one K/V tile read serves all of them.
#include "pa_device.h"

// ring items of a suffix item (K and V of PA_SUFFIX_DEPTH / 2 groups in flight); one
// group ahead measured best on the shared-prefix batch (57.3 us; two 57.7, three 58.2)
#ifndef PA_SUFFIX_DEPTH
#define PA_SUFFIX_DEPTH 2
#endif

namespace {

// Shared prefix (parallel sampling, shared prompts): the leading tokens a group of
// sequences shares are read once for all of them, and each member's own tokens once for
// that member. Both kinds of work are a row item: the rows of `members` consecutive
// sequences from `first` (M = members x G query rows, the columns of the score tiles; set
// s holds rows 16 s .. 16 s + 15, zero past M) over tokens [t0, t0 + ntok), read through
// the block table of `first` (for a prefix item every member's table holds the same blocks
// there), so each K and V tile feeds every member. Scores: v_mfma_f32_16x16x32_bf16, lane
// (r, c) then holds tokens r + 4i of query row 16 s + c; online softmax per column; PV:
// v_mfma_f32_16x16x16_bf16 with those probabilities (rounded to bf16) as A, leaving lane
// (r, c) with query rows 16 s + 4 r + i of output columns c * EV .. c * EV + EV - 1. Every
// (member, head) gets a partial record in slot `slot` (slot < 0: the row's only partition,
// written normalized to `out`); the partition merge combines the prefix and own-token
// records. DEPTH ring items: K and V of DEPTH / 2 groups ahead of the
// consumer, K and V of a group issued together.
template <int D, int NSET, int DEPTH>
__device__ __forceinline__ void row_item(const Params& p, int g, int first, int members, int t0,
                                         int ntok, int slot) {
    constexpr int ROW = D * 2;
    constexpr int NQ = D / 32;
    constexpr int WV = D / 8;
    constexpr int EV = D / 16;
    constexpr int U = DEPTH / 2;
    static_assert(D == 64 || D == 128, "head size");
    static_assert(DEPTH >= 2 && DEPTH % 2 == 0, "ring holds whole groups (K and V)");

    const int lane = threadIdx.x & 63;
    const int G = p.Hq / p.Hkv;
    const int M = members * G;           // query rows (host checks M <= 16 * NSET)
    const int part = slot;
    const int ng = (ntok + 15) >> 4;
    const int last = ng - 1;

    // table entries of the partition's groups, read from the first member's row
    int tblv;
    {
        const int32_t* trow = p.tables + (int64_t)first * p.max_blocks;
        int i = (t0 + lane * 16) >> p.bs_shift;
        i = i < p.max_blocks ? i : p.max_blocks - 1;
        const int e = trow[i];
        tblv = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
    }
    const int r = lane >> 4;
    const int c = lane & 15;
    u32x4_t qf[NSET][NQ];
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        const int qr = 16 * s + c;
        if (qr < M) {
            const int mb = qr / G, hh = qr - mb * G;
            const char* qrow = p.q + ((int64_t)(first + mb) * p.Hq + g * G + hh) * ROW;
#pragma unroll
            for (int k = 0; k < NQ; ++k)
                qf[s][k] = *reinterpret_cast<const u32x4_t*>(qrow + (k * 32 + r * 8) * 2);
        } else {
#pragma unroll
            for (int k = 0; k < NQ; ++k) qf[s][k] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    const int64_t tile_bytes = (int64_t)p.bs * ROW;
    const int64_t blk_bytes = (int64_t)p.Hkv * tile_bytes;
    const int bs_mask = p.bs - 1;
    const char* kbase = p.k + g * tile_bytes;
    const char* vbase = p.v + g * tile_bytes;
    const uint32_t koff = (uint32_t)(((c >> 2) + 4 * (c & 3)) * ROW + r * 16);
    const uint32_t voff = (uint32_t)(r * ROW + c * WV);
    struct Item {
        u32x4_t q[NQ];
    };
    // groups past the partition (the ring runs two ahead) read the head's first tile
    // instead: never used, and it stays in cache (the loads are non-temporal)
    auto goff = [&](int gq) -> int64_t {
        if (gq > last) return 0;
        const int ph = __builtin_amdgcn_readlane(tblv, gq);
        return (int64_t)ph * blk_bytes + (int64_t)((t0 + gq * 16) & bs_mask) * ROW;
    };
    auto issue_k = [&](int gq, Item& dst) {
        const char* kb = kbase + goff(gq);
#pragma unroll
        for (int k = 0; k < NQ; ++k) dst.q[k] = ld16<PA_PREFIX_NT != 0>(reinterpret_cast<const u32x4_t*>(kb + koff + k * 64));
    };
    auto issue_v = [&](int gq, Item& dst) {
        const char* vb = vbase + goff(gq);
        if constexpr (WV == 16) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                dst.q[k] = ld16<PA_PREFIX_NT != 0>(reinterpret_cast<const u32x4_t*>(vb + voff + k * 4 * ROW));
        } else {
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                const u32x2_t a = *reinterpret_cast<const u32x2_t*>(vb + voff + k * 4 * ROW);
                const u32x2_t e = *reinterpret_cast<const u32x2_t*>(vb + voff + (k + 1) * 4 * ROW);
                dst.q[k / 2] = __builtin_shufflevector(a, e, 0, 1, 2, 3);
            }
        }
    };
    auto vword = [&](const Item& it, int k, int w) -> uint32_t {
        if constexpr (WV == 16) return it.q[k][w];
        else return it.q[k >> 1][(k & 1) * 2 + w];
    };

    f32x4_t acc[NSET][EV];
    float m_run[NSET], l_run[NSET];
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        m_run[s] = -INFINITY;
        l_run[s] = 0.f;
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[s][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float cl2 = p.scale_log2;
    Item ring[DEPTH];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        issue_k(u, ring[2 * u]);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(u, ring[2 * u + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);

    for (int t0g = 0; t0g < ng; t0g += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0g + u;
            Item& kit = ring[2 * u];
            Item& vit = ring[2 * u + 1];
            const bool live = t < ng;
            const int valid = min(16, ntok - 16 * t);
            float y[NSET][4];
            uint32_t pw[NSET][2];
            if (live) {
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < NQ; ++k)
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, kit.q[k]),
                            __builtin_bit_cast(bf16x8_t, qf[s][k]), sc, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[s][i] = sc[i] * cl2;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            issue_k(t + U, kit);
            __builtin_amdgcn_sched_barrier(0);
            if (live) {
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    if (valid < 16) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) y[s][i] = (r + 4 * i < valid) ? y[s][i] : -INFINITY;
                    }
                    const float mx = fmaxf(fmaxf(y[s][0], y[s][1]), fmaxf(y[s][2], y[s][3]));
                    const float m_new = fmaxf(m_run[s], rows_max(mx));
                    const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);   // per column
                    m_run[s] = m_new;
                    // output rows 4r + i of this lane take the factor of column 4r + i
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float ai = col_bcast(alpha, i);
#pragma unroll
                        for (int e = 0; e < EV; ++e) acc[s][e][i] *= ai;
                    }
                    const bf16x2_t p01 = __builtin_convertvector(
                        (f32x2_t){__builtin_amdgcn_exp2f(y[s][0] - m_new), __builtin_amdgcn_exp2f(y[s][1] - m_new)}, bf16x2_t);
                    const bf16x2_t p23 = __builtin_convertvector(
                        (f32x2_t){__builtin_amdgcn_exp2f(y[s][2] - m_new), __builtin_amdgcn_exp2f(y[s][3] - m_new)}, bf16x2_t);
                    pw[s][0] = __builtin_bit_cast(uint32_t, p01);
                    pw[s][1] = __builtin_bit_cast(uint32_t, p23);
                    l_run[s] = l_run[s] * alpha + ((lo_bf16(pw[s][0]) + hi_bf16(pw[s][0])) +
                                                   (lo_bf16(pw[s][1]) + hi_bf16(pw[s][1])));
                }
                if (valid < 16) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        if (r + 4 * k >= valid) {
                            if constexpr (WV == 16) {
                                vit.q[k] = u32x4_t{0u, 0u, 0u, 0u};
                            } else {
                                vit.q[k >> 1][(k & 1) * 2] = 0u;
                                vit.q[k >> 1][(k & 1) * 2 + 1] = 0u;
                            }
                        }
                    }
                }
#pragma unroll
                for (int w = 0; w < WV / 4; ++w) {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t sel = h ? 0x07060302u : 0x05040100u;
                        const u32x2_t bv = {__builtin_amdgcn_perm(vword(vit, 1, w), vword(vit, 0, w), sel),
                                            __builtin_amdgcn_perm(vword(vit, 3, w), vword(vit, 2, w), sel)};
#pragma unroll
                        for (int s = 0; s < NSET; ++s) {
                            const u32x2_t av = {pw[s][0], pw[s][1]};
                            acc[s][2 * w + h] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                                __builtin_bit_cast(s16x4_t, av), __builtin_bit_cast(s16x4_t, bv),
                                acc[s][2 * w + h], 0, 0, 0);
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            issue_v(t + U, vit);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // records: query row qr = 16 s + 4 r + i sits in lane (r, c), output columns c*EV..;
    // its (max, sum) were kept per column qr
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        const float lcol = rows_sum(l_run[s]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qr = 16 * s + 4 * r + i;
            const float lr = __shfl(lcol, 4 * r + i);
            const float mr = __shfl(m_run[s], 4 * r + i);
            if (qr < M) {
                const int mb = qr / G, hh = qr - mb * G;
                const int64_t row = (int64_t)(first + mb) * p.Hq + g * G + hh;
                if (slot < 0) {        // the row's only partition: the normalized output
                    const float inv = 1.0f / lr;
                    float* dst = p.out + row * D + c * EV;
#pragma unroll
                    for (int e = 0; e < EV; e += 4)
                        *reinterpret_cast<float4*>(dst + e) =
                            make_float4(acc[s][e][i] * inv, acc[s][e + 1][i] * inv,
                                        acc[s][e + 2][i] * inv, acc[s][e + 3][i] * inv);
                } else {
                    float* dst = p.ws_o + (row * p.n_parts + part) * D + c * EV;
#pragma unroll
                    for (int e = 0; e < EV; e += 4)
                        *reinterpret_cast<float4*>(dst + e) =
                            make_float4(acc[s][e][i], acc[s][e + 1][i], acc[s][e + 2][i], acc[s][e + 3][i]);
                    if (c == 0) p.ws_ml[row * p.n_parts + part] = make_float2(mr, lr);
                }
            }
        }
    }
}

// A prefix item: (group, KV head, partition of pre_tokens shared tokens). Its ring runs
// one group ahead: the suffix items that run beside these waves are short and bound by
// chains of dependent reads, and a shallower ring here leaves them more of the memory
// system (2 groups ahead measured 59.2 us on the shared-prefix batch, 1 group 58.3,
// 4 groups 62.8).
template <int D, int NSET>
__device__ __forceinline__ void prefix_item(const Params& p, int id) {
    const int g = id % p.Hkv;
    const int rest = id / p.Hkv;
    const int gi_ = rest % p.n_groups;
    const int part = rest / p.n_groups;
    const int first = p.groups[3 * gi_];
    int members = p.groups[3 * gi_ + 1];
    members = members > p.max_members ? p.max_members : members;
    members = members > p.B - first ? p.B - first : members;   // stay inside the batch
    const int cap = p.max_blocks * p.bs;
    int shared_tok = p.groups[3 * gi_ + 2];
    shared_tok = (shared_tok > p.max_shared ? p.max_shared : shared_tok) & ~15;   // whole groups
    shared_tok = shared_tok < 0 ? 0 : (shared_tok > cap ? cap : shared_tok);
    const int t0 = part * p.pre_tokens;
    if (first < 0 || first >= p.B || t0 >= shared_tok || members <= 0) return;
    row_item<D, NSET, 2>(p, g, first, members, t0, min(p.pre_tokens, shared_tok - t0), part);
}

// A suffix item: (sequence, KV head, partition of part_tokens of the sequence's own
// tokens, those after its group's shared prefix). One member, G query rows in one column
// set; K and V of a group are loaded together, so a short row costs few dependent round
// trips. Records go to the slots after the sequence's prefix
// partitions; a partition past the sequence's end leaves nothing.
// With no groups at all the launch is a plain partitioned decode: a row with one partition
// is written normalized, an empty row as zeros, and only longer rows leave records.
template <int D>
__device__ __forceinline__ void suffix_item(const Params& p, int id) {
    int g, b, part;
    work_item(p, id, g, b, part);
    const int cap = p.max_blocks * p.bs;
    int L = p.lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const bool plain = p.groups == nullptr;
    const int start = plain ? 0 : min(group_shared(p, b), L);
    const int slot0 = (start + p.pre_tokens - 1) / p.pre_tokens;
    const int t0 = start + part * p.part_tokens;
    if (t0 >= L) {
        if (plain && part == 0) {   // empty sequence: a zero row per head
            const int G = p.Hq / p.Hkv;
            for (int i = (int)(threadIdx.x & 63); i < G * D; i += 64)
                p.out[((int64_t)b * p.Hq + g * G) * D + i] = 0.f;
        }
        return;
    }
    const int slot = plain && L <= p.part_tokens ? -1 : slot0 + part;
    row_item<D, 1, PA_SUFFIX_DEPTH>(p, g, b, 1, t0, min(p.part_tokens, L - t0), slot);
}

// Multi-query attention with a causal mask (prefill, a chunk of a long prompt, draft
// tokens): the last n_b tokens of sequence b are queries at once, query j at position
// p_j = L_b - n_b + j seeing tokens 0 .. p_j. One wavefront per (KV head, query tile,
// token partition, sequence). A query tile is 16 NSET of the sequence's n_b x G query rows
// (row = j G + head, so consecutive rows of a token share its position); they are the
// columns of the score tiles as in prefix_item, so each K and V tile read serves the whole
// tile. The partition covers tokens [part P, (part + 1) P) up to the tile's last position;
// a group that reaches past the tile's first position is masked per column (a select, so
// poison never leaks). The table entries of 64 groups at a time sit in one VGPR.
// A row whose position lies in partition 0 (np = 1) is written normalized; otherwise
// every partition leaves a record and multi rows are merged by decode_reduce_kernel.
template <int D, int NSET>
__device__ __forceinline__ void multi_item(const Params& p, int g, int b, int part, int tile) {
    constexpr int ROW = D * 2;
    constexpr int NQ = D / 32;
    constexpr int WV = D / 8;
    constexpr int EV = D / 16;
    constexpr int DEPTH = 4;             // ring items: K and V of two groups
    constexpr int U = DEPTH / 2;
    static_assert(D == 64 || D == 128, "head size");

    const int lane = threadIdx.x & 63;
    if (b >= p.B) return;
    const int cap = p.max_blocks * p.bs;
    int L = p.lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    int qs, n;
    multi_rows(p, b, L, &qs, &n);
    const int G = p.Hq / p.Hkv;
    const int row0 = tile * 16 * NSET;
    const int M = min(16 * NSET, n * G - row0);   // query rows of this tile
    if (M <= 0) return;
    const int base = L - n;                        // position of the chunk's first query
    const int pos_first = base + row0 / G;
    const int pos_last = base + (row0 + M - 1) / G;
    const int P = p.part_tokens;
    const int t0 = part * P;
    if (t0 > pos_last) return;
    const int ntok = min(pos_last + 1, t0 + P) - t0;
    const int ng = (ntok + 15) >> 4;
    const int last = ng - 1;

    // table entries of groups 64w .. 64w + 63 of the partition, lane i holding group 64w + i
    const int32_t* trow = p.tables + (int64_t)b * p.max_blocks;
    auto load_window = [&](int w) -> int {
        int i = (t0 + (w * 64 + lane) * 16) >> p.bs_shift;
        i = i < p.max_blocks ? i : p.max_blocks - 1;
        const int e = trow[i];
        return e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
    };
    int tblv = load_window(0);
    int win = 0;

    const int r = lane >> 4;
    const int c = lane & 15;
    u32x4_t qf[NSET][NQ];
    int pos_c[NSET];                     // position of column c of set s (-1 past the tile)
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        const int qr = 16 * s + c;
        if (qr < M) {
            const int row = row0 + qr;
            const int j = row / G, hh = row - j * G;
            pos_c[s] = base + j;
            const char* qrow = p.q + ((int64_t)(qs + j) * p.Hq + g * G + hh) * ROW;
#pragma unroll
            for (int k = 0; k < NQ; ++k)
                qf[s][k] = *reinterpret_cast<const u32x4_t*>(qrow + (k * 32 + r * 8) * 2);
        } else {
            pos_c[s] = -1;
#pragma unroll
            for (int k = 0; k < NQ; ++k) qf[s][k] = u32x4_t{0u, 0u, 0u, 0u};
        }
    }

    const int64_t tile_bytes = (int64_t)p.bs * ROW;
    const int64_t blk_bytes = (int64_t)p.Hkv * tile_bytes;
    const int bs_mask = p.bs - 1;
    const char* kbase = p.k + g * tile_bytes;
    const char* vbase = p.v + g * tile_bytes;
    const uint32_t koff = (uint32_t)(((c >> 2) + 4 * (c & 3)) * ROW + r * 16);
    const uint32_t voff = (uint32_t)(r * ROW + c * WV);
    struct Item {
        u32x4_t q[NQ];
    };
    auto goff = [&](int gq) -> int64_t {
        gq = gq < last ? gq : last;
        const int w = gq >> 6;
        if (w != win) {
            // a new window of table entries (every 64 groups): the ring drains once
            win = w;
            tblv = load_window(w);
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
        }
        const int ph = __builtin_amdgcn_readlane(tblv, gq & 63);
        return (int64_t)ph * blk_bytes + (int64_t)((t0 + gq * 16) & bs_mask) * ROW;
    };
    auto issue_k = [&](int gq, Item& dst) {
        const char* kb = kbase + goff(gq);
#pragma unroll
        for (int k = 0; k < NQ; ++k) dst.q[k] = *reinterpret_cast<const u32x4_t*>(kb + koff + k * 64);
    };
    auto issue_v = [&](int gq, Item& dst) {
        const char* vb = vbase + goff(gq);
        if constexpr (WV == 16) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                dst.q[k] = *reinterpret_cast<const u32x4_t*>(vb + voff + k * 4 * ROW);
        } else {
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                const u32x2_t a = *reinterpret_cast<const u32x2_t*>(vb + voff + k * 4 * ROW);
                const u32x2_t e = *reinterpret_cast<const u32x2_t*>(vb + voff + (k + 1) * 4 * ROW);
                dst.q[k / 2] = __builtin_shufflevector(a, e, 0, 1, 2, 3);
            }
        }
    };
    auto vword = [&](const Item& it, int k, int w) -> uint32_t {
        if constexpr (WV == 16) return it.q[k][w];
        else return it.q[k >> 1][(k & 1) * 2 + w];
    };

    f32x4_t acc[NSET][EV];
    // the softmax sums of output rows 4r + i, accumulated on the matrix cores as P times
    // a column of ones (the same rounded probabilities the PV product uses)
    f32x4_t lsum[NSET];
    float m_run[NSET];
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};   // bf16 1.0
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        m_run[s] = -INFINITY;
        lsum[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[s][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    const float cl2 = p.scale_log2;
    Item ring[DEPTH];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        __builtin_amdgcn_sched_barrier(0);
        issue_k(u, ring[2 * u]);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(u, ring[2 * u + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);

    // scores of one group for every set: y[s][o + i] for tokens r + 4i of the group. The
    // sets' accumulations are interleaved (head-dim chunk outer, set inner), so NSET
    // independent products are in flight instead of one dependent chain.
    auto qk = [&](const Item& kit, float (&y)[NSET][8], int o) {
        f32x4_t sc[NSET];
#pragma unroll
        for (int s = 0; s < NSET; ++s) sc[s] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
#pragma unroll
            for (int s = 0; s < NSET; ++s)
                sc[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, kit.q[k]),
                    __builtin_bit_cast(bf16x8_t, qf[s][k]), sc[s], 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i) y[s][o + i] = sc[s][i] * cl2;
        }
    };
    // rows past `valid` of a V item may hold anything: their probabilities are 0, their
    // values are zeroed too
    auto zero_rows = [&](Item& vit, int valid) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (r + 4 * k >= valid) {
                if constexpr (WV == 16) {
                    vit.q[k] = u32x4_t{0u, 0u, 0u, 0u};
                } else {
                    vit.q[k >> 1][(k & 1) * 2] = 0u;
                    vit.q[k >> 1][(k & 1) * 2 + 1] = 0u;
                }
            }
        }
    };

    // Two groups (32 tokens) per step: both score tiles, one online-softmax update, and PV
    // on v_mfma_f32_16x16x32_bf16 whose k index runs over the 8 tokens a lane holds (r + 4i
    // of the first group, then of the second), for the probabilities and V alike.
    for (int t = 0; t < ng; t += 2) {
        Item& k0 = ring[0];
        Item& v0 = ring[1];
        Item& k1 = ring[2];
        Item& v1 = ring[3];
        const bool live1 = t + 1 < ng;
        const int tg = t0 + 16 * t;              // first token of the pair
        float y[NSET][8];
        qk(k0, y, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue_k(t + 2, k0);
        __builtin_amdgcn_sched_barrier(0);
        qk(k1, y, 4);                            // a re-read of the last group when !live1
        __builtin_amdgcn_sched_barrier(0);
        issue_k(t + 3, k1);
        __builtin_amdgcn_sched_barrier(0);
        // the causal edge, the partition's end or a missing second group fall in this pair
        const bool edge = tg + 31 > pos_first || !live1;
        if (edge) {
#pragma unroll
            for (int s = 0; s < NSET; ++s) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int tok = tg + (i >> 2) * 16 + r + 4 * (i & 3);
                    const bool ok = tok <= pos_c[s] && (i < 4 || live1);
                    y[s][i] = ok ? y[s][i] : -INFINITY;
                }
            }
        }
        // m_run is each column's reference, not always its maximum: it moves (and the
        // accumulators are rescaled) only when some column's maximum passes its reference
        // by more than PA_LAZY_RESCALE (log2 units), so the probabilities stay below
        // 2^PA_LAZY_RESCALE. Softmax does not depend on the reference, and a column that
        // has seen no token yet moves at its first token. A column with no token keeps
        // m = -inf and 0 as the exponent reference, so its factors are 0.
        // A column's maximum passes its reference exactly when one of the four lanes that
        // hold the column has a score past it, so the common step tests each lane's own
        // maximum (one ballot for all sets, no cross-lane reduction) and the column maxima
        // are formed only when some set moves; the decision is still per set.
        float mx[NSET];
        bool move = false;
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            mx[s] = y[s][0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx[s] = __builtin_elementwise_maximum(mx[s], y[s][i]);
            move = move || mx[s] > m_run[s] + (float)PA_LAZY_RESCALE;
        }
        if (__ballot(move) != 0) {
#pragma unroll
            for (int s = 0; s < NSET; ++s) {
                const float m_new = fmaxf(m_run[s], rows_max(mx[s]));
                if (__ballot(m_new > m_run[s] + (float)PA_LAZY_RESCALE) != 0) {
                    const float m_to = m_new == -INFINITY ? 0.f : m_new;
                    const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_to);   // per column
                    m_run[s] = m_new;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float ai = col_bcast(alpha, i);
#pragma unroll
                        for (int e = 0; e < EV; ++e) acc[s][e][i] *= ai;
                        lsum[s][i] *= ai;
                    }
                }
            }
        }
        uint32_t pw[NSET][4];
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            const float m_ref = m_run[s] == -INFINITY ? 0.f : m_run[s];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const bf16x2_t pp = __builtin_convertvector(
                    (f32x2_t){__builtin_amdgcn_exp2f(y[s][2 * w] - m_ref),
                              __builtin_amdgcn_exp2f(y[s][2 * w + 1] - m_ref)}, bf16x2_t);
                pw[s][w] = __builtin_bit_cast(uint32_t, pp);
            }
            const u32x4_t av = {pw[s][0], pw[s][1], pw[s][2], pw[s][3]};
            lsum[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, ones), lsum[s], 0, 0, 0);
        }
        if (edge) {
            zero_rows(v0, ntok - 16 * t);
            zero_rows(v1, live1 ? ntok - 16 * (t + 1) : 0);
        }
        // every V operand first (its own registers), so the 8 NSET products that follow
        // issue back to back instead of waiting to overwrite the operand the previous
        // products still read
        u32x4_t bv[WV / 4][2];
#pragma unroll
        for (int w = 0; w < WV / 4; ++w) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t sel = h ? 0x07060302u : 0x05040100u;
                bv[w][h] = u32x4_t{__builtin_amdgcn_perm(vword(v0, 1, w), vword(v0, 0, w), sel),
                                   __builtin_amdgcn_perm(vword(v0, 3, w), vword(v0, 2, w), sel),
                                   __builtin_amdgcn_perm(vword(v1, 1, w), vword(v1, 0, w), sel),
                                   __builtin_amdgcn_perm(vword(v1, 3, w), vword(v1, 2, w), sel)};
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_v(t + 2, v0);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(t + 3, v1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int w = 0; w < WV / 4; ++w) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    const u32x4_t av = {pw[s][0], pw[s][1], pw[s][2], pw[s][3]};
                    acc[s][2 * w + h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv[w][h]),
                        acc[s][2 * w + h], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }

    // output row qr = 16 s + 4 r + i sits in lane (r, c), columns c*EV..; its maximum was
    // kept per column qr, its sum in lsum[s][i]
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qr = 16 * s + 4 * r + i;
            const float lr = lsum[s][i];
            const float mr = __shfl(m_run[s], 4 * r + i);
            if (qr < M) {
                const int row = row0 + qr;
                const int j = row / G, hh = row - j * G;
                const int pos = base + j;
                if (pos >= t0) {
                    const int64_t grow = (int64_t)(qs + j) * p.Hq + g * G + hh;
                    if (pos < P) {                  // the row's only partition
                        const float inv = 1.0f / lr;
                        float* dst = p.out + grow * D + c * EV;
#pragma unroll
                        for (int e = 0; e < EV; e += 4)
                            *reinterpret_cast<float4*>(dst + e) =
                                make_float4(acc[s][e][i] * inv, acc[s][e + 1][i] * inv,
                                            acc[s][e + 2][i] * inv, acc[s][e + 3][i] * inv);
                    } else {
                        float* dst = p.ws_o + (grow * p.n_parts + part) * D + c * EV;
#pragma unroll
                        for (int e = 0; e < EV; e += 4)
                            *reinterpret_cast<float4*>(dst + e) =
                                make_float4(acc[s][e][i], acc[s][e + 1][i], acc[s][e + 2][i], acc[s][e + 3][i]);
                        if (c == 0) p.ws_ml[grow * p.n_parts + part] = make_float2(mr, lr);
                    }
                }
            }
        }
    }
}

// Longest-first order of the multi-query work.
//
// A unit is (sequence b, token partition part, query tile t); its Hkv items (one per KV
// head) are adjacent in the grid. Its work is ntok, the tokens of the partition that the
// tile's last query sees. Waves take units in decreasing ntok, counted in classes of
// 2^lpt_shift tokens (class k holds ntok in ((k-1)Q, kQ], the last class everything above),
// and within a class by sequence, then partition, then tile from the last. Longest first
// keeps a long unit from starting last behind a CU that already ran short ones; the classes
// keep a sequence's neighbouring tiles together so they share the XCD's L2. The order moves
// work between waves only: every unit's arithmetic, and so every output bit, is the same
// in any order.
//
// Each block derives the order itself: the per-sequence query counts go to LDS, every
// (sequence, partition) pair adds its tiles to the class histogram, a scan turns the
// histogram into class starts, and each wave finds its unit from its rank: the class by a
// binary search, then the pair by a running count over the pairs in order, then the tile.
// Tiles of a sequence with n queries after `base` cached tokens see, for tile t,
// vis(t) = base + (min((t+1) R, n G) - 1) / G + 1 tokens (R = 16 NSET rows per tile);
// vis increases with t, so the tiles with vis >= y are the last tiles_from(y) ones.
constexpr int kLptBuckets = 1024;
constexpr int kLptSeqs = 2048;

__device__ __forceinline__ int tiles_from(int y, int base, int n, int nt, int G, int rshift) {
    const int d = y - base - 1;
    if (d < 0) return nt;
    if (n <= d) return 0;
    return nt + 1 - ((d * G + (1 << rshift)) >> rshift);   // nt - (ceil((dG + 1) / R) - 1)
}

// Tiles of pair (b, part) in class k: the last `a` tiles hold ntok > (k-1)Q, the last
// `c` of those ntok > kQ (c = 0 in the top class).
__device__ __forceinline__ void class_tiles(int k, int part, int base, int n, int nt, int G, int rshift,
                                            const Params& p, int* a, int* c) {
    const int lo = part * p.part_tokens + ((k - 1) << p.lpt_shift);
    *a = tiles_from(lo + 1, base, n, nt, G, rshift);
    *c = k < p.lpt_buckets ? tiles_from(lo + (1 << p.lpt_shift) + 1, base, n, nt, G, rshift) : 0;
}

// The unit of rank `rank` in the longest-first order; false when rank is past the last
// unit. Every thread of the block calls it (it holds block barriers).
template <int NSET>
__device__ bool lpt_unit(const Params& p, int rank, int* b_out, int* part_out, int* tile_out) {
    __shared__ int2 seq[kLptSeqs];          // (cached tokens before the chunk, queries)
    __shared__ int hist[kLptBuckets];       // units per class, top class first
    __shared__ int start[kLptBuckets];      // their exclusive prefix
    constexpr int rshift = 4 + (NSET == 1 ? 0 : (NSET == 2 ? 1 : 2));
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int G = p.Hq / p.Hkv;
    const int K = p.lpt_buckets;
    const int P = p.part_tokens;
    const int cap = p.max_blocks * p.bs;
    for (int i = tid; i < K; i += 256) hist[i] = 0;
    for (int b = tid; b < p.B; b += 256) {
        int L = p.lens[b];
        L = L < 0 ? 0 : (L > cap ? cap : L);
        int qs, n;
        multi_rows(p, b, L, &qs, &n);
        seq[b] = make_int2(L - n, n);
    }
    __syncthreads();
    const int NP = p.B * p.n_parts;
    for (int pr = tid; pr < NP; pr += 256) {
        const int b = pr / p.n_parts, part = pr - b * p.n_parts;
        const int base = seq[b].x, n = seq[b].y;
        const int L = base + n;
        if (n <= 0 || part * P >= L) continue;
        const int nt = (n * G + (16 * NSET - 1)) >> rshift;
        // ntok of the pair's first tile (the one with the fewest tokens) and of its last
        const int tf = nt - tiles_from(part * P + 1, base, n, nt, G, rshift);
        const int vf = base + (min((tf + 1) << rshift, n * G) - 1) / G + 1;
        const int k_lo = (min(vf, (part + 1) * P) - part * P + (1 << p.lpt_shift) - 1) >> p.lpt_shift;
        const int k_hi = (min(L, (part + 1) * P) - part * P + (1 << p.lpt_shift) - 1) >> p.lpt_shift;
        for (int k = k_lo; k <= k_hi; ++k) {
            int a, c;
            class_tiles(k, part, base, n, nt, G, rshift, p, &a, &c);
            if (a > c) atomicAdd(&hist[K - k], a - c);
        }
    }
    __syncthreads();
    if (tid < 64) {
        // exclusive scan of the histogram: lane i sums a run of slots, the lanes' totals
        // are scanned across the wave, then each lane writes its run
        const int per = (K + 63) >> 6;
        const int s0 = min(lane * per, K), s1 = min(s0 + per, K);
        int run = 0;
        for (int s = s0; s < s1; ++s) run += hist[s];
        int incl = run;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            incl += lane >= d ? o : 0;
        }
        int acc = incl - run;
        for (int s = s0; s < s1; ++s) {
            start[s] = acc;
            acc += hist[s];
        }
    }
    __syncthreads();
    const int total = start[K - 1] + hist[K - 1];
    if (rank >= total) return false;
    int lo = 0, hi = K - 1;                 // last slot whose start is <= rank
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (start[mid] <= rank) lo = mid;
        else hi = mid - 1;
    }
    const int k = K - lo;
    int j = rank - start[lo];
    for (int c0 = 0; c0 < NP; c0 += 64) {
        const int pr = c0 + lane;
        int cnt = 0, a = 0, c = 0;
        if (pr < NP) {
            const int b = pr / p.n_parts, part = pr - b * p.n_parts;
            const int base = seq[b].x, n = seq[b].y;
            if (n > 0 && part * P < base + n) {
                const int nt = (n * G + (16 * NSET - 1)) >> rshift;
                class_tiles(k, part, base, n, nt, G, rshift, p, &a, &c);
                cnt = a > c ? a - c : 0;
            }
        }
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(incl, d);
            incl += lane >= d ? o : 0;
        }
        const int sum = __shfl(incl, 63);
        if (j < sum) {
            const uint64_t m = __ballot(incl > j);
            const int w = __builtin_ctzll(m);
            const int before = __shfl(incl - cnt, w);
            const int cw = __shfl(c, w);
            const int prw = c0 + w;
            const int b = prw / p.n_parts;
            const int n = seq[b].y;
            const int nt = (n * G + (16 * NSET - 1)) >> rshift;
            *b_out = b;
            *part_out = prw - b * p.n_parts;
            *tile_out = nt - cw - 1 - (j - before);   // tiles from the last within the class
            return true;
        }
        j -= sum;
    }
    return false;
}

// All multi-query items, four per 256-thread block.
template <int D, int NSET>
__global__ __launch_bounds__(256) void decode_multi_kernel(Params p) {
    const int item = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (int)(threadIdx.x >> 6));
    const int g = item % p.Hkv;
    int b, part, tile;
    if (p.lpt_buckets > 0) {
        if (!lpt_unit<NSET>(p, item / p.Hkv, &b, &part, &tile)) return;
        b = __builtin_amdgcn_readfirstlane(b);
        part = __builtin_amdgcn_readfirstlane(part);
        tile = __builtin_amdgcn_readfirstlane(tile);
    } else {
        // grid order: KV head fastest (the heads spread over the XCDs), then query tile from
        // the last (a chunk's later tiles see the most tokens, so they start first), then
        // partition, then sequence
        if (item >= p.pre_items) return;
        int rest = item / p.Hkv;
        tile = p.n_tiles - 1 - rest % p.n_tiles;
        rest /= p.n_tiles;
        part = rest % p.n_parts;
        b = rest / p.n_parts;
    }
    multi_item<D, NSET>(p, g, b, part, tile);
}

// The prefix partitions and the members' own tokens in one launch of 4-wave blocks, one
// item per wave: blocks below pre_blocks hold the prefix items (first, so that the longest
// work starts earliest), the rest the suffix partitions. A suffix partition is short (the
// tokens a member added after the shared prefix), so it gets a single wave and a small
// chunk, which starts its V loads after four K tiles rather than eight.
template <int D, int G, int NSET>
__global__ __launch_bounds__(256) void decode_shared_kernel(Params p) {
    const int bid = blockIdx.x;
    const int item = __builtin_amdgcn_readfirstlane((bid < p.pre_blocks ? bid : bid - p.pre_blocks) * 4 + (int)(threadIdx.x >> 6));
    if (bid < p.pre_blocks) {
        if (item < p.pre_items) prefix_item<D, NSET>(p, item);
    } else if (item < p.suf_items) {
        suffix_item<D>(p, item);
    }
}

template <int D, int G>
hipError_t launch_fused(const Params& prm, int nset, int n_suf, hipStream_t s) {
    const dim3 grid(prm.pre_blocks + (prm.suf_items + 3) / 4);
    if (nset == 1) hipLaunchKernelGGL((decode_shared_kernel<D, G, 1>), grid, dim3(256), 0, s, prm);
    else if (nset == 2) hipLaunchKernelGGL((decode_shared_kernel<D, G, 2>), grid, dim3(256), 0, s, prm);
    else hipLaunchKernelGGL((decode_shared_kernel<D, G, 4>), grid, dim3(256), 0, s, prm);
    return hipSuccess;
}

template <int D>
hipError_t launch_shared_d(Params prm, int G, int nset, int n_pre, int n_suf, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    prm.pre_items = prm.n_groups * prm.Hkv * n_pre;
    prm.pre_blocks = (prm.pre_items + 3) / 4;
    prm.suf_items = n_suf * prm.Hkv * prm.B;
    hipError_t e;
    switch (G) {
        case 1: e = launch_fused<D, 1>(prm, nset, n_suf, s); break;
        case 2: e = launch_fused<D, 2>(prm, nset, n_suf, s); break;
        case 4: e = launch_fused<D, 4>(prm, nset, n_suf, s); break;
        case 8: e = launch_fused<D, 8>(prm, nset, n_suf, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3((prm.Hq * prm.B + 3) / 4), dim3(256), 0, s, prm);
    return hipGetLastError();
}

template <int D>
hipError_t launch_multi_d(const Params& prm, int nset, hipStream_t s) {
    const dim3 grid((prm.pre_items + 3) / 4);
    if (nset == 1) hipLaunchKernelGGL((decode_multi_kernel<D, 1>), grid, dim3(256), 0, s, prm);
    else if (nset == 2) hipLaunchKernelGGL((decode_multi_kernel<D, 2>), grid, dim3(256), 0, s, prm);
    else hipLaunchKernelGGL((decode_multi_kernel<D, 4>), grid, dim3(256), 0, s, prm);
    if (prm.n_parts > 1)
        hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3((prm.Hq * prm.total_q + 3) / 4), dim3(256), 0, s, prm);
    return hipGetLastError();
}

}  // namespace

namespace pa_internal {

int launch_decode_shared(const SharedLaunch& a, const char** err) {
    Params prm{};
    prm.out = a.out;
    prm.ws_o = a.ws_o;
    prm.ws_ml = reinterpret_cast<float2*>(a.ws_ml);
    prm.q = static_cast<const char*>(a.q);
    prm.k = static_cast<const char*>(a.k);
    prm.v = static_cast<const char*>(a.v);
    prm.tables = a.tables;
    prm.lens = a.lens;
    prm.B = a.B;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.bs = a.bs;
    int shift = 0;
    while ((1 << shift) < a.bs) ++shift;
    prm.bs_shift = shift;
    prm.num_blocks = a.num_blocks;
    prm.max_blocks = a.max_blocks;
    prm.part_tokens = a.part_tokens;
    prm.n_parts = a.n_slots;
    prm.scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    prm.groups = a.groups;
    prm.n_groups = a.n_groups;
    prm.pre_tokens = a.pre_tokens;
    prm.max_members = a.max_members;
    prm.max_shared = a.max_shared;
    if (a.B == 0) return 0;
    const int G = a.Hq / a.Hkv;
    const int m = a.max_members * G;
    const int nset = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
    const hipError_t e = a.D == 64 ? launch_shared_d<64>(prm, G, nset, a.n_pre, a.n_suf, a.stream)
                       : a.D == 128 ? launch_shared_d<128>(prm, G, nset, a.n_pre, a.n_suf, a.stream)
                                    : hipErrorInvalidValue;
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

int launch_decode_multi(const MultiLaunch& a, const char** err) {
    if (a.stream_g > 0) return launch_multi_stream(a, err);
    Params prm{};
    prm.out = a.out;
    prm.ws_o = a.ws_o;
    prm.ws_ml = reinterpret_cast<float2*>(a.ws_ml);
    prm.q = static_cast<const char*>(a.q);
    prm.k = static_cast<const char*>(a.k);
    prm.v = static_cast<const char*>(a.v);
    prm.tables = a.tables;
    prm.lens = a.lens;
    prm.B = a.B;
    prm.Hq = a.Hq;
    prm.Hkv = a.Hkv;
    prm.bs = a.bs;
    int shift = 0;
    while ((1 << shift) < a.bs) ++shift;
    prm.bs_shift = shift;
    prm.num_blocks = a.num_blocks;
    prm.max_blocks = a.max_blocks;
    prm.part_tokens = a.part_tokens;
    prm.n_parts = a.n_parts;
    prm.scale_log2 = (float)((double)a.scale * 1.4426950408889634);
    prm.q_starts = a.q_starts;
    prm.total_q = a.total_q;
    prm.max_q = a.max_q;
    prm.n_tiles = a.n_tiles;
    prm.pre_items = a.Hkv * a.n_tiles * a.n_parts * a.B;   // host-checked to fit
    // work classes of 256 tokens (more per class for partitions beyond 256k tokens)
    int qsh = 8;
    while (((a.part_tokens + (1 << qsh) - 1) >> qsh) > kLptBuckets) ++qsh;
    prm.lpt_shift = qsh;
    prm.lpt_buckets = (a.longest_first && a.B <= kLptSeqs) ? (a.part_tokens + (1 << qsh) - 1) >> qsh : 0;
    if (a.B == 0 || a.total_q == 0) return 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(a.stream);
    const hipError_t e = a.D == 64 ? launch_multi_d<64>(prm, a.nset, s)
                       : a.D == 128 ? launch_multi_d<128>(prm, a.nset, s)
                                    : hipErrorInvalidValue;
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

}  // namespace pa_internal
