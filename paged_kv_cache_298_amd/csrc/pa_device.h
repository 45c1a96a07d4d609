// pa_device.h -- device code shared by the decode kernels (pa_decode.hip) and the
// shared-prefix and multi-query kernels (pa_multi.hip): the kernel parameter block, the
// cross-lane helpers, the bf16 partition item and the partition merge kernel. For HIP
// translation units only; everything sits in an anonymous namespace, so each unit
// compiles its own copy of what it uses.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pa_internal.h"

// Build-time tuning knobs: ring depth (16-token groups in flight per wave) of the bf16 and
// fp32 kernels, and whether the bf16 kernel computes a ring's groups back to back before
// refilling them.
#ifndef PA_BF16_DEPTH
#define PA_BF16_DEPTH 4
#endif
#ifndef PA_BF16_CHUNK
#define PA_BF16_CHUNK 8
#endif
#ifndef PA_BF16_QLDS
#define PA_BF16_QLDS 0
#endif
#ifndef PA_BF16_WAVES
#define PA_BF16_WAVES 4
#endif
#ifndef PA_STREAM_DEPTH
#define PA_STREAM_DEPTH 4
#endif
// G = 8 decode in the stream kernel: one set of 8 distinct head columns (repeated twice)
// rather than two sets of 4 heads repeated four times (half the matrix and softmax work)
#ifndef PA_STREAM_DIST8
#define PA_STREAM_DIST8 1
#endif
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 4
#endif
// Prefill / prompt-chunk tiles: the softmax reference of a query column moves only when
// its maximum passes it by more than this many log2 units (0: at every new maximum).
#ifndef PA_LAZY_RESCALE
#define PA_LAZY_RESCALE 8
#endif

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediate for vmcnt(0) with the other counters left free (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm0 = 0x0F70;

struct Params {
    float* out;
    float* ws_o;
    float2* ws_ml;
    const char* q;
    const char* k;
    const char* v;
    const int32_t* tables;
    const int32_t* lens;
    int B, Hq, Hkv, bs, bs_shift, num_blocks, max_blocks, part_tokens, n_parts;
    float scale_log2;
    // stream decomposition only
    float* rec_o;     // [2 * nw, G, D] partial outputs of rows a wave covers only in part
    float2* rec_ml;   // [2 * nw, G]    their (max in log2 units, sum)
    int4* desc;       // [nw] first row of each wave's slice: b, g, row start, row groups
    int* meta;        // [2] groups in the stream, waves given a slice
    int nw;           // waves launched
    int min_slice;    // fewest 16-token groups per wave
    // shared-prefix decomposition only (groups == nullptr otherwise)
    const int32_t* groups;   // [n_groups, 3]: first sequence, members, shared tokens; sorted
    int n_groups;
    int pre_tokens;          // tokens per prefix partition
    int max_members;         // host bounds the device groups are clamped to (they size the
    int max_shared;          // workspace and the query tiles)
    int pre_items;           // prefix items (group, KV head, partition) of a fused launch
    int pre_blocks;          // blocks holding them, four items each
    int suf_items;           // suffix partitions of a fused launch
    // fused cache write (pa_decode_append) only: the newest token of every sequence, K and
    // V rows [B, Hkv, D], and its slot (< 0: none); read from here for position L - 1
    const char* nkey;
    const char* nval;
    const int32_t* nslots;
    // multi-query mode only (q_starts == nullptr otherwise)
    const int32_t* q_starts; // [B + 1] offsets of each sequence's queries in q
    int total_q;             // query tokens in q (host value the device offsets are clamped to)
    int max_q;               // host bound on queries per sequence
    int n_tiles;             // query tiles per (sequence, KV head)
    int lpt_buckets;         // work classes of the longest-first order (0: grid order)
    int lpt_shift;           // log2 of the tokens per work class
};

// Shared-prefix mode: the tokens sequence b shares with its group (groups are sorted by
// first sequence and disjoint), rounded down to whole 16-token groups and clamped to the
// host bound; 0 when b is in no group. The caller clamps it to b's length. Called by all
// 64 lanes of a wave with the same b: a 64-way search in which each lane tests one
// candidate per step, so up to 64 groups cost one memory round trip and up to 4096 two (a
// binary search would pay one per halving). Members are clamped to the host bound, as
// the prefix kernel clamps them.
__device__ __forceinline__ int group_shared(const Params& p, int b) {
    const int lane = threadIdx.x & 63;
    int lo = 0, n = p.n_groups;   // candidates lo .. lo + n - 1
    int found = -1, first = 0, members = 0, sh = 0;
    while (n > 0) {
        const int stride = (n + 63) >> 6;
        const bool in = lane * stride < n;
        const int32_t* gp = p.groups + 3 * (lo + (in ? lane * stride : 0));
        int f = gp[0], mm = gp[1], ss = gp[2];
        // all three fields arrive in one round trip: keep the compiler from deferring the
        // loads of the two used only once a candidate is found
        asm volatile("" : "+v"(f), "+v"(mm), "+v"(ss));
        const uint64_t m = __ballot(in && f <= b);
        if (m == 0) break;
        const int k = 63 - __builtin_clzll(m);           // last candidate starting <= b
        found = lo + k * stride;
        first = __builtin_amdgcn_readlane(f, k);
        members = __builtin_amdgcn_readlane(mm, k);
        sh = __builtin_amdgcn_readlane(ss, k);
        if (stride == 1) break;
        const int end = lo + n;
        lo = found + 1;
        n = min(stride - 1, end - lo);
    }
    members = members > p.max_members ? p.max_members : members;
    if (found < 0 || b < first || b - first >= members) return 0;
    sh = (sh > p.max_shared ? p.max_shared : sh) & ~15;   // whole 16-token groups only
    return sh < 0 ? 0 : sh;
}

// Multi-query mode: the first query row qs of sequence b and its query count n, clamped
// so that 0 <= n <= min(L, max_q) and qs + n <= total_q (offsets that break the
// preconditions give wrong rows, never an access outside q or out).
__device__ __forceinline__ void multi_rows(const Params& p, int b, int L, int* qs, int* n) {
    int s = p.q_starts[b];
    const int e = p.q_starts[b + 1];
    s = s < 0 ? 0 : (s > p.total_q ? p.total_q : s);
    int k = e - s;
    k = k < 0 ? 0 : k;
    k = min(k, min(L, p.max_q));
    k = min(k, p.total_q - s);
    *qs = s;
    *n = k;
}

// Multi-query mode: the sequence whose queries include global query qi, i.e. the last b
// with q_starts[b] <= qi (0 if none). All 64 lanes of a wave call it with the same qi;
// the same 64-way search as group_shared.
__device__ __forceinline__ int seq_of_query(const Params& p, int qi) {
    const int lane = threadIdx.x & 63;
    int lo = 0, n = p.B, found = 0;
    while (n > 0) {
        const int stride = (n + 63) >> 6;
        const bool in = lane * stride < n;
        const int f = p.q_starts[lo + (in ? lane * stride : 0)];
        const uint64_t m = __ballot(in && f <= qi);
        if (m == 0) break;
        found = lo + (63 - __builtin_clzll(m)) * stride;
        if (stride == 1) break;
        const int end = lo + n;
        lo = found + 1;
        n = min(stride - 1, end - lo);
    }
    return found;
}

__device__ __forceinline__ float lo_bf16(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// 16 x 16 score tile: rows = the 16 tokens of a group, columns = query heads (G used).
// Lane l holds rows 4*(l/16) + i (i = 0..3) of column l % 16 on return.
template <bool BF16, int KL>
__device__ __forceinline__ f32x4_t qk_tile(const u32x4_t (&kf)[KL], const u32x4_t (&qf)[KL]) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
#pragma unroll
        for (int c = 0; c < KL; ++c)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kf[c]),
                                                          __builtin_bit_cast(bf16x8_t, qf[c]),
                                                          acc, 0, 0, 0);
    } else {
#pragma unroll
        for (int c = 0; c < KL; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(kf[c][j]),
                                                           __uint_as_float(qf[c][j]), acc, 0, 0,
                                                           0);
    }
    return acc;
}

#ifndef PA_DECODE_NT
#define PA_DECODE_NT 0
#endif

// The stream kernel's K/V tile loads carry the non-temporal hint: every K/V byte is read
// once per call, and streaming it past the caches raised the Llama-3-8B batch from 5.1 to
// 6.0 TB/s (a cache policy only; the data are the same).
#ifndef PA_STREAM_NT
#define PA_STREAM_NT 1
#endif
__device__ __forceinline__ u32x4_t kv_load16(const u32x4_t* ptr) {
#if PA_STREAM_NT
    return __builtin_nontemporal_load(ptr);
#else
    return *ptr;
#endif
}

// Non-temporal K/V loads of the bf16 partition item (partition decode) and of the
// shared-prefix row items, each read once per call.
#ifndef PA_ITEM_NT
#define PA_ITEM_NT 1
#endif
#ifndef PA_PREFIX_NT
#define PA_PREFIX_NT 1
#endif
template <bool NT>
__device__ __forceinline__ u32x4_t ld16(const u32x4_t* ptr) {
    if constexpr (NT) return __builtin_nontemporal_load(ptr);
    else return *ptr;
}

// K/V bytes are read once per call: stream them past the caches when PA_DECODE_NT is set.
__device__ __forceinline__ u32x4_t load16(const u32x4_t* ptr) {
#if PA_DECODE_NT
    return __builtin_nontemporal_load(ptr);
#else
    return *ptr;
#endif
}

// The workgroup is exactly one wavefront, so LDS traffic between its lanes needs only
// ordering, not a workgroup barrier: LDS instructions of one wave execute in issue order.
// Wavefront-scope fences keep the compiler from reordering across this point and, unlike
// a workgroup barrier, do not wait for outstanding global loads.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Work item of this workgroup. The grid is one-dimensional and ordered KV head fastest,
// then sequence, then partition. Consecutive workgroups are dealt round-robin to the
// eight XCDs, each of which has its own L2 and its own link to HBM, so this order gives
// every XCD the same mix of heads, sequences and partitions: with 8 KV heads, XCD k serves
// KV head k of every partition, an exact eighth of the bytes. (Partition-fastest order
// would send every sequence's first partition, the one that always exists, to one XCD.)
__device__ __forceinline__ void work_item(const Params& p, int id, int& g, int& b, int& part) {
    g = id % p.Hkv;
    const int rest = id / p.Hkv;
    b = rest % p.B;
    part = rest / p.B;
}

template <int G>
__device__ __forceinline__ void load_probs(const float* __restrict__ src, float (&p)[G]) {
    if constexpr (G % 4 == 0) {
#pragma unroll
        for (int h = 0; h < G; h += 4) {
            const float4 x = *reinterpret_cast<const float4*>(src + h);
            p[h] = x.x; p[h + 1] = x.y; p[h + 2] = x.z; p[h + 3] = x.w;
        }
    } else if constexpr (G == 2) {
        const float2 x = *reinterpret_cast<const float2*>(src);
        p[0] = x.x; p[1] = x.y;
    } else {
#pragma unroll
        for (int h = 0; h < G; ++h) p[h] = src[h];
    }
}

// ---------------------------------------------------------------------------------------
// bf16 caches: one pass per partition, K and V of each 16-token group loaded together,
// both contractions on the matrix cores.
//
// QK^T: v_mfma_f32_16x16x32_bf16 with A = the 16 K rows of the group and B = query heads.
// MFMA row m = 4r + i carries token r + 4i (r = lane / 16 of the lane feeding that row
// is not the same r; the permutation only decides which row each lane loads), and the 16
// columns carry the group's 4 heads of a head set, each repeated 4 times. Then lane
// (r = lane / 16, c = lane % 16) receives in register i the score of token r + 4i for head
// c % 4, which is exactly the A operand that v_mfma_f32_4x4x1_16b_f32 (16 blocks of
// 4 x 4 x 1) needs for PV: block lanes 4b..4b+3 (all of row group r) supply
// p[head lane % 4][token r + 4i] and, as B, one element of V row r + 4i, the element a
// coalesced 16-byte load of that row already holds. PV therefore needs no transpose, no
// LDS and no cross-lane exchange; the four row groups' partial sums are added at the end.
//
// Work is done in chunks of kChunk groups (128 tokens): the chunk's kChunk QK^T MFMA
// chains are independent, then one online-softmax update per head (new running maximum,
// accumulators and running sum multiplied by exp2(old max - new max), a factor that is
// exactly 1 when the maximum did not move), then the chunk's PV MFMAs. The loads form one
// stream in consumption order, K of the chunk's groups then V of the same groups, held in
// a ring of DEPTH items of equal size, so DEPTH - 1 items are in flight while one is used.

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

template <int W> struct VecOf;
template <> struct VecOf<16> { typedef u32x4_t type; };
template <> struct VecOf<8> { typedef u32x2_t type; };

// Sum / max over the four 16-lane row groups without LDS traffic: gfx950's permlane swaps
// exchange the odd rows (16 lanes) / the upper half (32 lanes) of one register with the
// even rows / lower half of another. Given two registers holding the same values, they
// then hold the row pairs (0,1),(2,3) crosswise, so one add or max completes a butterfly
// step. Both registers are outputs of the instruction, so it is written as inline
// assembly with two read-write operands (preceded by the wait states a VALU result needs
// before a permlane reads it).
__device__ __forceinline__ void swap_rows16(uint32_t& a, uint32_t& b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_halves(uint32_t& a, uint32_t& b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float rows_sum(float v) {
    uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
    swap_rows16(a, b);
    uint32_t c = __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
    uint32_t d = c;
    swap_halves(c, d);
    return __builtin_bit_cast(float, c) + __builtin_bit_cast(float, d);
}
__device__ __forceinline__ float rows_max(float v) {
    uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
    swap_rows16(a, b);
    uint32_t c = __builtin_bit_cast(uint32_t, fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b)));
    uint32_t d = c;
    swap_halves(c, d);
    return fmaxf(__builtin_bit_cast(float, c), __builtin_bit_cast(float, d));
}
// value of lane (lane & ~3) + m of the same quad, via DPP
__device__ __forceinline__ float quad_bcast(float v, int m) {
    const int x = __builtin_bit_cast(int, v);
    int y;
    switch (m) {
        case 0: y = __builtin_amdgcn_mov_dpp(x, 0x00, 0xf, 0xf, false); break;
        case 1: y = __builtin_amdgcn_mov_dpp(x, 0x55, 0xf, 0xf, false); break;
        case 2: y = __builtin_amdgcn_mov_dpp(x, 0xaa, 0xf, 0xf, false); break;
        default: y = __builtin_amdgcn_mov_dpp(x, 0xff, 0xf, 0xf, false); break;
    }
    return __builtin_bit_cast(float, y);
}

// Value held by column 4r + m, for a lane of row group r (lanes 16r .. 16r + 15), when all
// four row groups hold the same per-column values (m a compile-time constant after
// unrolling). Four DPP row broadcasts (lane n of every 16-lane row to the whole row),
// each written only to the row group that needs it: no LDS round trip, unlike a lane
// shuffle.
#ifndef PA_COL_DPP
#define PA_COL_DPP 1
#endif
template <int M>
__device__ __forceinline__ int col_bcast_m(int x) {
    int y = x;
    y = __builtin_amdgcn_update_dpp(y, x, 0x150 + M, 0x1, 0xf, false);
    y = __builtin_amdgcn_update_dpp(y, x, 0x150 + 4 + M, 0x2, 0xf, false);
    y = __builtin_amdgcn_update_dpp(y, x, 0x150 + 8 + M, 0x4, 0xf, false);
    y = __builtin_amdgcn_update_dpp(y, x, 0x150 + 12 + M, 0x8, 0xf, false);
    return y;
}
__device__ __forceinline__ float col_bcast(float v, int m) {
#if PA_COL_DPP
    const int x = __builtin_bit_cast(int, v);
    int y;
    switch (m) {
        case 0: y = col_bcast_m<0>(x); break;
        case 1: y = col_bcast_m<1>(x); break;
        case 2: y = col_bcast_m<2>(x); break;
        default: y = col_bcast_m<3>(x); break;
    }
    return __builtin_bit_cast(float, y);
#else
    return __shfl(v, 4 * ((int)(threadIdx.x & 63) >> 4) + m);
#endif
}

template <int D, int G, int DEPTH, int kChunk, bool QLDS, int W>
__device__ __forceinline__ void bf16_item(const Params& p, int id) {
    constexpr int ROW = D * 2;              // bytes per cached row
    constexpr int NQ = D / 32;              // 16-byte registers per ring item
    constexpr int WV = D / 8;               // bytes of a V row per lane per load (16 or 8)
    constexpr int EV = D / 16;              // bf16 elements per lane per V load
    constexpr int NSET = (G + 3) / 4;       // head sets of 4
    constexpr int G4 = G < 4 ? G : 4;       // distinct heads in a set
    constexpr int ITEMS = 2 * kChunk;       // ring items per chunk: K groups, then V groups
    typedef typename VecOf<WV>::type vload_t;
    static_assert(D == 64 || D == 128, "head size");
    static_assert(kChunk % DEPTH == 0, "the ring depth must divide the chunk");

    const int lane = threadIdx.x & 63;
    const int wid = W == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave in the group
    int g, b, part;
    work_item(p, id, g, b, part);
    const int cap = p.max_blocks * p.bs;
    int L = p.lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int hq0 = g * G;
    const int t0 = part * p.part_tokens;
    // Wave wid takes the partition's 16-token groups wid, wid + W, wid + 2W, ... (its
    // "local" groups 0, 1, 2, ...). The block-table entries of those groups are fetched
    // before the sequence length is known (they do not depend on it): lane i holds the
    // entry of local group i, clamped into the row and into the pool, and the loop reads
    // it with v_readlane.
    int tblv;
    {
        const int32_t* trow = p.tables + (int64_t)b * p.max_blocks;
        int i = (t0 + (wid + lane * W) * 16) >> p.bs_shift;
        i = i < p.max_blocks ? i : p.max_blocks - 1;
        const int e = trow[i];
        tblv = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
    }
    if (t0 >= L) {
        if (part == 0) {   // empty sequence: a zero row per head
            for (int i = threadIdx.x; i < G * D; i += 64 * W)
                p.out[((int64_t)b * p.Hq + hq0) * D + i] = 0.f;
        }
        return;
    }
    const int ntok_part = min(p.part_tokens, L - t0);
    const int ng_part = (ntok_part + 15) >> 4;
    // this wave's stream: ngroups local groups, all full but possibly the last, which
    // holds the partition's final tokens; ntok counts the stream's tokens
    const int ngroups = ng_part > wid ? (ng_part - wid + W - 1) / W : 0;
    const int last = ngroups - 1;
    const int ntok = ngroups > 0 ? last * 16 + min(16, ntok_part - (wid + last * W) * 16) : 0;
    const int nchunks = (ngroups + kChunk - 1) / kChunk;
    const int nparts_b = (L + p.part_tokens - 1) / p.part_tokens;
    const int slot = part;

    const int r = lane >> 4;     // row group
    const int c = lane & 15;     // column
    // query fragments, B operand of QK: column c of set s is head 4s + (c % 4) % G4; held
    // in registers, or (QLDS) parked in LDS and re-read per group to save registers
    u32x4_t qf[QLDS ? 1 : NSET][QLDS ? 1 : NQ];
    __shared__ u32x4_t q_lds[QLDS ? NSET * NQ * 64 : 1];
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        const int h = 4 * s + ((c & 3) % G4);
        const char* qrow = p.q + ((int64_t)b * p.Hq + hq0 + h) * ROW;
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
            const u32x4_t x = *reinterpret_cast<const u32x4_t*>(qrow + (k * 32 + r * 8) * 2);
            if constexpr (QLDS) q_lds[(s * NQ + k) * 64 + lane] = x;
            else qf[s][k] = x;
        }
    }
    auto qfrag = [&](int s, int k) -> u32x4_t {
        if constexpr (QLDS) return q_lds[(s * NQ + k) * 64 + lane];
        else return qf[s][k];
    };
    if constexpr (QLDS) wave_sync();

    const int64_t tile_bytes = (int64_t)p.bs * ROW;              // one (block, head) tile
    const int64_t blk_bytes = (int64_t)p.Hkv * tile_bytes;       // one physical block
    const char* kbase = p.k + g * tile_bytes;
    const char* vbase = p.v + g * tile_bytes;
    const int bs_mask = p.bs - 1;
    // K: lane feeds MFMA row c, i.e. token (c / 4) + 4 (c % 4) of the group, 16 bytes at
    // 64 k + 16 r; V: row r (+4 per load), bytes c * WV of the row
    const uint32_t koff = (uint32_t)(((c >> 2) + 4 * (c & 3)) * ROW + r * 16);
    const uint32_t voff = (uint32_t)(r * ROW + c * WV);

    struct Item {
        u32x4_t q[NQ];
    };
    // load stream item t of chunk ch (t < kChunk: K of group t, else V of group t - kChunk);
    // groups past the partition are clamped to its last group (a re-read that hits in cache)
    // slots past the stream's last group (the last chunk's tail) read the first tile of
    // the head instead: the data are never used, and that tile stays in cache, where a
    // re-read of the last group would fetch it from HBM again (non-temporal loads)
    auto issue = [&](int ch, int t, Item& dst) {
        const bool is_v = t >= kChunk;
        int gi = ch * kChunk + (is_v ? t - kChunk : t);
        const bool past = gi > last;
        gi = gi < last ? gi : last;
        const int ph = __builtin_amdgcn_readlane(tblv, gi);
        const int tok = t0 + (wid + gi * W) * 16;
        const int64_t off = past ? 0 : (int64_t)ph * blk_bytes + (int64_t)(tok & bs_mask) * ROW;
        if (!is_v) {
            const char* kb = kbase + off;
#pragma unroll
            for (int k = 0; k < NQ; ++k)
                dst.q[k] = ld16<PA_ITEM_NT != 0>(reinterpret_cast<const u32x4_t*>(kb + koff + k * 64));
        } else {
            const char* vb = vbase + off;
            if constexpr (WV == 16) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    dst.q[k] = ld16<PA_ITEM_NT != 0>(reinterpret_cast<const u32x4_t*>(vb + voff + k * 4 * ROW));
            } else {
#pragma unroll
                for (int k = 0; k < 4; k += 2) {
                    const u32x2_t a = *reinterpret_cast<const u32x2_t*>(vb + voff + k * 4 * ROW);
                    const u32x2_t e = *reinterpret_cast<const u32x2_t*>(vb + voff + (k + 1) * 4 * ROW);
                    dst.q[k / 2] = __builtin_shufflevector(a, e, 0, 1, 2, 3);
                }
            }
        }
    };
    // dword w of V load k within an item
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

    // One chunk: consume its 2 * kChunk stream items in order, refilling each ring slot
    // with the item DEPTH positions later. `masked` (the last chunk only) handles tokens
    // past the end of the partition and groups past its last one.
    auto chunk = [&](int ch, bool masked) {
        float y[NSET][kChunk][4];   // scores in log2 units, then probabilities
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
            Item& it = ring[t % DEPTH];
            if (t < kChunk) {
                // ---- scores of group t on the matrix cores
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k = 0; k < NQ; ++k)
                        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, it.q[k]),
                            __builtin_bit_cast(bf16x8_t, qfrag(s, k)), sc, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[s][t][i] = sc[i] * cl2;
                }
                if (t == kChunk - 1) {
                    // ---- one online-softmax update for the chunk's 128 tokens
                    const int tc = ch * kChunk * 16;   // first token of the chunk
#pragma unroll
                    for (int s = 0; s < NSET; ++s) {
                        if (masked) {
#pragma unroll
                            for (int u = 0; u < kChunk; ++u)
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    y[s][u][i] = (tc + u * 16 + r + 4 * i < ntok) ? y[s][u][i] : -INFINITY;
                        }
                        float mx = y[s][0][0];
#pragma unroll
                        for (int u = 0; u < kChunk; ++u)
#pragma unroll
                            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, y[s][u][i]);
                        const float m_new = fmaxf(m_run[s], rows_max(mx));
                        const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_new);
                        m_run[s] = m_new;
                        float am[4];
#pragma unroll
                        for (int m = 0; m < 4; ++m) am[m] = quad_bcast(alpha, m);
#pragma unroll
                        for (int e = 0; e < EV; ++e)
#pragma unroll
                            for (int m = 0; m < 4; ++m) acc[s][e][m] *= am[m];
                        float ls = 0.f;
#pragma unroll
                        for (int u = 0; u < kChunk; ++u) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float e2 = __builtin_amdgcn_exp2f(y[s][u][i] - m_new);
                                y[s][u][i] = masked ? ((y[s][u][i] == -INFINITY) ? 0.f : e2) : e2;
                            }
                            ls += (y[s][u][0] + y[s][u][1]) + (y[s][u][2] + y[s][u][3]);
                        }
                        l_run[s] = l_run[s] * alpha + ls;
                    }
                }
            } else {
                // ---- o += p * V for group u on the matrix cores
                const int u = t - kChunk;
                const int gi = ch * kChunk + u;
                bool skip = false;
                if (masked) {
                    skip = gi > last;
                    if (!skip && gi == last) {   // rows past the end may hold anything
                        const int tl = gi * 16;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            if (tl + r + 4 * k >= ntok) {
                                if constexpr (WV == 16) {
                                    it.q[k] = u32x4_t{0u, 0u, 0u, 0u};
                                } else {
                                    it.q[k >> 1][(k & 1) * 2] = 0u;
                                    it.q[k >> 1][(k & 1) * 2 + 1] = 0u;
                                }
                            }
                        }
                    }
                }
                if (!skip) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
#pragma unroll
                        for (int w = 0; w < WV / 4; ++w) {
                            const uint32_t uw = vword(it, k, w);
                            const float v0 = lo_bf16(uw), v1 = hi_bf16(uw);
#pragma unroll
                            for (int s = 0; s < NSET; ++s) {
                                acc[s][2 * w] = __builtin_amdgcn_mfma_f32_4x4x1f32(y[s][u][k], v0, acc[s][2 * w], 0, 0, 0);
                                acc[s][2 * w + 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(y[s][u][k], v1, acc[s][2 * w + 1], 0, 0, 0);
                            }
                        }
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            issue(ch + (t + DEPTH) / ITEMS, (t + DEPTH) % ITEMS, it);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (ngroups > 0) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) issue(0, j, ring[j]);
        for (int ch = 0; ch < nchunks - 1; ++ch) chunk(ch, false);
        chunk(nchunks - 1, true);
    }

    // add the four row groups' partial sums (lanes c, c + 16, c + 32, c + 48)
#pragma unroll
    for (int s = 0; s < NSET; ++s) {
        l_run[s] = rows_sum(l_run[s]);
#pragma unroll
        for (int e = 0; e < EV; ++e)
#pragma unroll
            for (int m = 0; m < 4; ++m) acc[s][e][m] = rows_sum(acc[s][e][m]);
    }
    // lane c (row group 0) now holds, for head m of each set, output columns
    // c*EV .. c*EV+EV-1; head m's sum and running maximum sit in quad lane m
    float lh[NSET][4], mh[NSET][4];
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            lh[s][m] = quad_bcast(l_run[s], m);
            mh[s][m] = quad_bcast(m_run[s], m);
        }
    if constexpr (W == 1) {
        if (r == 0) {
#pragma unroll
            for (int s = 0; s < NSET; ++s) {
#pragma unroll
                for (int m = 0; m < G4; ++m) {
                    const int h = 4 * s + m;
                    float o[EV];
#pragma unroll
                    for (int e = 0; e < EV; ++e) o[e] = acc[s][e][m];
                    if (nparts_b == 1) {
                        const float inv = 1.0f / lh[s][m];
                        float* dst = p.out + ((int64_t)b * p.Hq + hq0 + h) * D + c * EV;
#pragma unroll
                        for (int e = 0; e < EV; e += 4)
                            *reinterpret_cast<float4*>(dst + e) =
                                make_float4(o[e] * inv, o[e + 1] * inv, o[e + 2] * inv, o[e + 3] * inv);
                    } else {
                        float* dst = p.ws_o + (((int64_t)b * p.Hq + hq0 + h) * p.n_parts + slot) * D + c * EV;
#pragma unroll
                        for (int e = 0; e < EV; e += 4)
                            *reinterpret_cast<float4*>(dst + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
                        if (c == 0)
                            p.ws_ml[((int64_t)b * p.Hq + hq0 + h) * p.n_parts + slot] =
                                make_float2(mh[s][m], lh[s][m]);
                    }
                }
            }
        }
    } else {
        // the W waves' partial states meet in LDS; every thread of the group then
        // combines one float4 of the G x D output exactly like the split reduce does
        __shared__ float4 o_lds[W][G][D / 4];
        __shared__ float2 ml_lds[W][G];
        if (r == 0) {
#pragma unroll
            for (int s = 0; s < NSET; ++s) {
#pragma unroll
                for (int m = 0; m < G4; ++m) {
                    const int h = 4 * s + m;
#pragma unroll
                    for (int e = 0; e < EV; e += 4)
                        o_lds[wid][h][(c * EV + e) / 4] =
                            make_float4(acc[s][e][m], acc[s][e + 1][m], acc[s][e + 2][m], acc[s][e + 3][m]);
                    if (c == 0) ml_lds[wid][h] = make_float2(mh[s][m], lh[s][m]);
                }
            }
        }
        __syncthreads();
        constexpr int C4 = D / 4;
        for (int i = threadIdx.x; i < G * C4; i += 64 * W) {
            const int h = i / C4, c4 = i % C4;
            float M = -INFINITY;
#pragma unroll
            for (int v = 0; v < W; ++v) M = fmaxf(M, ml_lds[v][h].x);
            float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
            float ls = 0.f;
#pragma unroll
            for (int v = 0; v < W; ++v) {
                const float2 ml = ml_lds[v][h];
                const float wgt = __builtin_amdgcn_exp2f(ml.x - M);   // 0 for an idle wave
                const float4 x = o_lds[v][h][c4];
                o.x += wgt * x.x; o.y += wgt * x.y; o.z += wgt * x.z; o.w += wgt * x.w;
                ls += wgt * ml.y;
            }
            const int64_t row = (int64_t)b * p.Hq + hq0 + h;
            if (nparts_b == 1) {
                const float inv = 1.0f / ls;
                reinterpret_cast<float4*>(p.out + row * D)[c4] =
                    make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
            } else {
                reinterpret_cast<float4*>(p.ws_o + (row * p.n_parts + slot) * D)[c4] = o;
                if (c4 == 0) p.ws_ml[row * p.n_parts + slot] = make_float2(M, ls);
            }
        }
    }
}

// Combine the partitions of one (sequence, query head):
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, with M = max_i m_i.
// One wave per row (four rows per workgroup, so a batch of rows takes few workgroups).
// Lane (pg, c4) folds partitions pg, pg + NPG, ... of float4 column c4, kB per batch,
// rescaling its running sum when the maximum grows; the NPG partial sums then meet by
// lane exchanges in a fixed order. The first batch is loaded before the partition count
// is known, together with the length (and group) that give it: slots below n_parts always
// lie in the row's workspace, and a slot past the count is dropped by a select, never
// weighted, since it may hold anything. Rows are (sequence, head), or (query, head) in
// multi-query mode; the launch covers ceil(rows / 4) workgroups.
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(Params p) {
    constexpr int C4 = D / 4;          // float4 columns (16 or 32)
    constexpr int NPG = 64 / C4;       // partition groups per wave (4 or 2)
    constexpr int kB = 8;              // partitions per group per batch
    const int lane = threadIdx.x & 63;
    const int c4 = lane % C4;
    const int pg = lane / C4;
    const int ny = p.q_starts != nullptr ? p.total_q : p.B;
    const int rid = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (rid >= ny * p.Hq) return;
    const int y = rid / p.Hq;          // the sequence, or in multi-query mode the query
    const int h = rid - y * p.Hq;
    const int64_t row = (int64_t)y * p.Hq + h;
    const float2* ml = p.ws_ml + row * p.n_parts;
    const float* wo = p.ws_o + row * p.n_parts * D;
    float2 mlv[kB];
    float4 ov[kB];
    auto load_batch = [&](int k0, int lim) {
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            int i = pg + NPG * (k0 + u);
            i = i < lim ? i : 0;
            mlv[u] = ml[i];
            ov[u] = reinterpret_cast<const float4*>(wo + (int64_t)i * D)[c4];
        }
    };
    // The first batch is loaded before the count is known. In shared-prefix mode it takes
    // the slots of a full prefix and one own partition (the other slots are there for the
    // table's capacity and mostly unused); a row with more records loads the rest below.
    const int spec = p.groups != nullptr
        ? min(p.n_parts, (p.max_shared + p.pre_tokens - 1) / p.pre_tokens + 1) : p.n_parts;
    load_batch(0, spec);

    const int cap = p.max_blocks * p.bs;
    int np;
    if (p.q_starts != nullptr) {
        // multi-query mode: query y of sequence b at position pos has pos / P + 1 partitions
        const int b = seq_of_query(p, y);
        int L = p.lens[b];
        L = L < 0 ? 0 : (L > cap ? cap : L);
        int qs, n;
        multi_rows(p, b, L, &qs, &n);
        const int j = y - qs;
        if (j < 0 || j >= n) return;
        np = (L - n + j) / p.part_tokens + 1;
        if (np <= 1) return;
    } else {
        const int b = y;
        // the length through a vector load (b copied into a VGPR) that the group search's
        // loads follow without a wait: a scalar load would be waited for first
        int bv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(bv) : "s"(b));
        const int L_raw = p.lens[bv];
        const int sh = p.groups != nullptr ? group_shared(p, b) : 0;
        const int L = L_raw < 0 ? 0 : (L_raw > cap ? cap : L_raw);
        if (p.groups != nullptr) {
            // shared-prefix mode: the prefix partitions of b's group, then b's own partitions,
            // all left as records (an empty sequence gets a zero row here)
            const int start = min(sh, L);
            np = (start + p.pre_tokens - 1) / p.pre_tokens + (L - start + p.part_tokens - 1) / p.part_tokens;
            if (np == 0) {
                for (int i = lane; i < D; i += 64) p.out[row * D + i] = 0.f;
                return;
            }
        } else {
            np = (L + p.part_tokens - 1) / p.part_tokens;
            if (np <= 1) return;
        }
    }

    if (np > spec) {
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int i = pg + NPG * u;
            if (i >= spec && i < np) {
                mlv[u] = ml[i];
                ov[u] = reinterpret_cast<const float4*>(wo + (int64_t)i * D)[c4];
            }
        }
    }

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f, m = -INFINITY;
    for (int k0 = 0; pg + NPG * k0 < np; k0 += kB) {
        if (k0 != 0) load_batch(k0, p.n_parts);
        float mn = m;
#pragma unroll
        for (int u = 0; u < kB; ++u)
            if (pg + NPG * (k0 + u) < np) mn = fmaxf(mn, mlv[u].x);
        const float a = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first batch
        acc.x *= a; acc.y *= a; acc.z *= a; acc.w *= a;
        den *= a;
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            if (pg + NPG * (k0 + u) < np) {
                const float w = __builtin_amdgcn_exp2f(mlv[u].x - mn);
                acc.x = fmaf(w, ov[u].x, acc.x);
                acc.y = fmaf(w, ov[u].y, acc.y);
                acc.z = fmaf(w, ov[u].z, acc.z);
                acc.w = fmaf(w, ov[u].w, acc.w);
                den = fmaf(w, mlv[u].y, den);
            }
        }
        m = mn;
    }
    // the partition groups meet pairwise (lane ^ C4, then lane ^ 2 C4); a group with no
    // partition holds m = -inf, so a pair of such groups takes 0 as its reference
#pragma unroll
    for (int st = C4; st < 64; st <<= 1) {
        const float om = __shfl_xor(m, st);
        const float od = __shfl_xor(den, st);
        const float4 oa = make_float4(__shfl_xor(acc.x, st), __shfl_xor(acc.y, st),
                                      __shfl_xor(acc.z, st), __shfl_xor(acc.w, st));
        const float M = fmaxf(m, om);
        const float Mr = M == -INFINITY ? 0.f : M;
        const float wa = __builtin_amdgcn_exp2f(m - Mr);
        const float wb = __builtin_amdgcn_exp2f(om - Mr);
        acc.x = acc.x * wa + oa.x * wb;
        acc.y = acc.y * wa + oa.y * wb;
        acc.z = acc.z * wa + oa.z * wb;
        acc.w = acc.w * wa + oa.w * wb;
        den = den * wa + od * wb;
        m = M;
    }
    if (pg == 0) {
        const float inv = 1.0f / den;
        reinterpret_cast<float4*>(p.out + row * D)[c4] =
            make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    }
}

}  // namespace
