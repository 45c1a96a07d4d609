// pa_decode.hip -- paged decode attention for gfx950 (MI355X).
//
// Sources: [P1] "PagedAttention" (inferensys.com glossary): the kernel reads the block
// table, gathers K/V from scattered physical blocks, handles a partly filled last block
// and fuses the gather into the attention; [P2] "Paged Attention" tutorial
// (infra.pidoku.co.in), section 5 "The kernel side": a loop over a sequence's blocks,
// phys = table[blk], q.k and an online softmax accumulated per block. That page's sketch
// and its cache layouts were written for NVIDIA warps; this file keeps what it computes
// and lays the work out for 64-lane CDNA4 wavefronts.
//
// Cache layout [num_blocks, Hkv, block_size, D]: a 16-token group of one KV head is one
// contiguous 16 x D tile of K and one of V. Every wavefront serves all G = Hq / Hkv query
// heads of its KV head, so each K/V byte is read from HBM once.
//
// Kernels:
//   decode_stream_kernel + stream_reduce_kernel (bf16 caches, the default): the batch's
//     (sequence, KV head) rows, cut into 16-token groups, are laid end to end and each
//     resident wavefront takes an equal contiguous slice; one load ring runs across row
//     boundaries; rows that cross slices leave partial states merged by the second kernel.
//   decode_bf16_kernel (bf16 fallback) and decode_partition_kernel (fp32): one workgroup
//     per (KV head, sequence, partition of P tokens); decode_reduce_kernel merges the
//     partitions.
// Scores: v_mfma_f32_16x16x32_bf16 (fp32: 16x16x4_f32) with the K tile as the A operand,
// each lane feeding token (c / 4) + 4 (c % 4) of its row group straight from one 16-byte
// load, and the G query rows (replicated to 16 columns) as B; lane (r, c) then holds
// tokens r + 4i of head column c. Softmax: online, in log2 units, masks by select (NaN in
// unused slots never leaks). PV: the stream kernel feeds those same registers (rounded to
// bf16) as the A operand of v_mfma_f32_16x16x16_bf16 against V rows gathered with byte
// permutes; the bf16 partition kernel uses v_mfma_f32_4x4x1_f32, the fp32 one the VALU.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

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
#ifndef PA_SHARED_DEPTH
#define PA_SHARED_DEPTH 4
#endif
#ifndef PA_SHARED_CHUNK
#define PA_SHARED_CHUNK 4
#endif
#ifndef PA_BF16_WAVES
#define PA_BF16_WAVES 4
#endif
#ifndef PA_STREAM_DEPTH
#define PA_STREAM_DEPTH 4
#endif
#ifndef PA_DECODE_DEPTH
#define PA_DECODE_DEPTH 4
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
    // multi-query mode only (q_starts == nullptr otherwise)
    const int32_t* q_starts; // [B + 1] offsets of each sequence's queries in q
    int total_q;             // query tokens in q (host value the device offsets are clamped to)
    int max_q;               // host bound on queries per sequence
    int n_tiles;             // query tiles per (sequence, KV head)
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

template <bool BF16, int D, int G, int DEPTH>
__global__ __launch_bounds__(64) void decode_partition_kernel(Params p) {
    constexpr int EB = BF16 ? 2 : 4;   // bytes per element
    constexpr int E = 16 / EB;         // elements per 16-byte load
    constexpr int KQ = D / 4;          // elements of a K row fed by one lane (quarter row)
    constexpr int NL = KQ / E;         // 16-byte loads per lane per 16-token group (K or V)
    constexpr int O = D / E;           // lanes covering one V row
    constexpr int R = 64 / O;          // V rows per wave-wide load
    constexpr int ROW = D * EB;        // bytes per cached row
    static_assert(NL >= 1 && R >= 1 && 16 / R == NL, "unsupported head size");

    extern __shared__ float smem[];
    float* s_lds = smem;                                            // [part_tokens][G]
    int* tbl = reinterpret_cast<int*>(smem + p.part_tokens * G);    // [part_tokens / 16]

    const int lane = threadIdx.x;
    int g, b, part;
    work_item(p, blockIdx.x, g, b, part);
    const int cap = p.max_blocks * p.bs;
    int L = p.lens[b];
    L = L < 0 ? 0 : (L > cap ? cap : L);
    const int t0 = part * p.part_tokens;
    const int hq0 = g * G;

    if (t0 >= L) {
        if (part == 0) {   // empty sequence: a zero row per head
            for (int i = lane; i < G * D; i += 64)
                p.out[((int64_t)b * p.Hq + hq0) * D + i] = 0.f;
        }
        return;
    }
    const int ntok = min(p.part_tokens, L - t0);
    const int ngroups = (ntok + 15) >> 4;
    const int nparts_b = (L + p.part_tokens - 1) / p.part_tokens;

    // block-table slice of this partition -> LDS (entries clamped into the pool)
    const int blk0 = t0 >> p.bs_shift;
    const int nblk = ((ntok - 1) >> p.bs_shift) + 1;
    const int32_t* trow = p.tables + (int64_t)b * p.max_blocks + blk0;
    for (int i = lane; i < nblk; i += 64) {
        int e = trow[i];
        e = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
        tbl[i] = e;
    }

    // Head-dim split of the QK contraction: MFMA step c takes elements
    // [c*4E, c*4E + 4E) of every row, lane quarter qd = lane / 16 the E of them at
    // c*4E + qd*E. Any split that A and B share gives the same dot products; this one makes
    // every K load instruction read 64 contiguous bytes of each of the 16 rows.
    // Query fragment: lane (column h = lane % 16, quarter qd) holds those elements of
    // q[b, hq0 + h, :]; zero for padded columns h >= G.
    const int col = lane & 15;
    const int qd = lane >> 4;
    u32x4_t qf[NL];
    if (col < G) {
        const char* qrow = p.q + ((int64_t)b * p.Hq + hq0 + col) * D * EB;
#pragma unroll
        for (int c = 0; c < NL; ++c)
            qf[c] = *reinterpret_cast<const u32x4_t*>(qrow + (c * 4 * E + qd * E) * EB);
    } else {
#pragma unroll
        for (int c = 0; c < NL; ++c) qf[c] = u32x4_t{0u, 0u, 0u, 0u};
    }
    wave_sync();

    // One stream of 2 * ngroups items: item i < ngroups is K group i, item ngroups + i is
    // V group i. Each item is NL 16-byte loads per lane; a ring of DEPTH items keeps
    // DEPTH * NL * 1 KiB in flight per wave, and V loads are already under way while
    // the softmax statistics of the partition are formed.
    const int64_t head_rows = (int64_t)p.bs;
    const int64_t blk_rows = (int64_t)p.Hkv * head_rows;
    const int bs_mask = p.bs - 1;
    const int lane_k_off = col * ROW + qd * 16;        // K: row `col`, piece `qd` (+64 B per load)
    const int vrow = lane / O;
    const int voct = lane % O;
    const int lane_v_off = vrow * ROW + voct * 16;     // V: row `vrow` (+R per load), slice voct
    const int nitems = 2 * ngroups;

    // Loads are issued unconditionally and in program order (past the end the index is
    // clamped to the last item, a re-read that hits in cache), so the compiler can keep
    // DEPTH - 1 items outstanding while it consumes one.
    auto issue = [&](int item, u32x4_t (&dst)[NL]) {
        item = item < nitems ? item : nitems - 1;
        const bool is_v = item >= ngroups;
        const int tl = (is_v ? item - ngroups : item) << 4;
        const int phys = __builtin_amdgcn_readfirstlane(tbl[tl >> p.bs_shift]);
        const int64_t row0 = (int64_t)phys * blk_rows + g * head_rows + (tl & bs_mask);
        const char* sbase = (is_v ? p.v : p.k) + row0 * ROW;
        const uint32_t voff = is_v ? lane_v_off : lane_k_off;
        const uint32_t vstride = is_v ? R * ROW : 64;
#pragma unroll
        for (int c = 0; c < NL; ++c)
            dst[c] = load16(reinterpret_cast<const u32x4_t*>(sbase + voff + c * vstride));
    };

    u32x4_t ring[DEPTH][NL];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) issue(j, ring[j]);

    float m_run = -INFINITY;
    float l_sum = 0.f;
    float acc[G][E];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;

    for (int i0 = 0; i0 < nitems; i0 += DEPTH) {
#pragma unroll
        for (int j = 0; j < DEPTH; ++j) {
            const int it = i0 + j;
            if (it < nitems) {
                if (it < ngroups) {
                    // ---- scores of K group `it` on the matrix cores
                    const int tl = it << 4;
                    const f32x4_t sc = qk_tile<BF16, NL>(ring[j], qf);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = tl + 4 * qd + i;
                        const float s = (t < ntok) ? sc[i] * p.scale_log2 : -INFINITY;
                        if (col < G) s_lds[t * G + col] = s;
                        m_run = fmaxf(m_run, s);
                    }
                    if (it == ngroups - 1) {
                        // ---- partition statistics: per-head max, p = exp2(s - m), sums
                        m_run = fmaxf(m_run, __shfl_xor(m_run, 16));
                        m_run = fmaxf(m_run, __shfl_xor(m_run, 32));
                        wave_sync();
                        const float m_mine = __shfl(m_run, lane % G);
                        const int nent = ngroups * 16 * G;
                        for (int e = lane; e < nent; e += 64) {
                            const float pe = __builtin_amdgcn_exp2f(s_lds[e] - m_mine);
                            s_lds[e] = pe;
                            l_sum += pe;
                        }
#pragma unroll
                        for (int off = G; off < 64; off <<= 1) l_sum += __shfl_xor(l_sum, off);
                        wave_sync();
                    }
                } else {
                    // ---- o += p * V for V group `it - ngroups` on the vector ALUs
                    const int tl = (it - ngroups) << 4;
                    if (tl + 16 > ntok) {   // last, partly valid group: zero rows past the end
#pragma unroll
                        for (int k = 0; k < NL; ++k)
                            if (tl + vrow + k * R >= ntok) ring[j][k] = u32x4_t{0u, 0u, 0u, 0u};
                    }
#pragma unroll
                    for (int k = 0; k < NL; ++k) {
                        float pk[G];
                        load_probs<G>(s_lds + (tl + vrow + k * R) * G, pk);
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const uint32_t u = ring[j][k][w];
                            if constexpr (BF16) {
                                const float x0 = lo_bf16(u), x1 = hi_bf16(u);
#pragma unroll
                                for (int h = 0; h < G; ++h) {
                                    acc[h][2 * w] = fmaf(pk[h], x0, acc[h][2 * w]);
                                    acc[h][2 * w + 1] = fmaf(pk[h], x1, acc[h][2 * w + 1]);
                                }
                            } else {
                                const float x = __uint_as_float(u);
#pragma unroll
                                for (int h = 0; h < G; ++h) acc[h][w] = fmaf(pk[h], x, acc[h][w]);
                            }
                        }
                    }
                }
            }
            issue(it + DEPTH, ring[j]);
        }
    }

    // sum the R row-groups that share a column slice
#pragma unroll
    for (int off = O; off < 64; off <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);

    float l_head[G];
#pragma unroll
    for (int h = 0; h < G; ++h) l_head[h] = __shfl(l_sum, h);

    if (nparts_b == 1) {
        if (vrow == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float inv = 1.0f / l_head[h];
                float* dst = p.out + ((int64_t)b * p.Hq + hq0 + h) * D + voct * E;
#pragma unroll
                for (int e = 0; e < E; e += 4)
                    *reinterpret_cast<float4*>(dst + e) =
                        make_float4(acc[h][e] * inv, acc[h][e + 1] * inv, acc[h][e + 2] * inv,
                                    acc[h][e + 3] * inv);
            }
        }
    } else {
        if (vrow == 0) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                float* dst = p.ws_o + (((int64_t)b * p.Hq + hq0 + h) * p.n_parts + part) * D +
                             voct * E;
#pragma unroll
                for (int e = 0; e < E; e += 4)
                    *reinterpret_cast<float4*>(dst + e) =
                        make_float4(acc[h][e], acc[h][e + 1], acc[h][e + 2], acc[h][e + 3]);
            }
        }
        if (lane < G) {   // lane h holds head h's max (col == h) and sum (h % G == h)
            p.ws_ml[((int64_t)b * p.Hq + hq0 + lane) * p.n_parts + part] = make_float2(m_run, l_sum);
        }
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
    // shared-prefix mode: this kernel covers only the tokens after the shared prefix and
    // always leaves partial records (slots after the prefix partitions)
    const bool shared = p.groups != nullptr;
    int start = 0, slot0 = 0;
    if (shared) {
        start = min(group_shared(p, b), L);
        slot0 = (start + p.pre_tokens - 1) / p.pre_tokens;
    }
    const int t0 = start + part * p.part_tokens;
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
        if (part == 0 && !shared) {   // empty sequence: a zero row per head
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
    const int nparts_b = shared ? 0 : (L + p.part_tokens - 1) / p.part_tokens;   // 0: records
    const int slot = slot0 + part;

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
    auto issue = [&](int ch, int t, Item& dst) {
        const bool is_v = t >= kChunk;
        int gi = ch * kChunk + (is_v ? t - kChunk : t);
        gi = gi < last ? gi : last;
        const int ph = __builtin_amdgcn_readlane(tblv, gi);
        const int tok = t0 + (wid + gi * W) * 16;
        const int64_t off = (int64_t)ph * blk_bytes + (int64_t)(tok & bs_mask) * ROW;
        if (!is_v) {
            const char* kb = kbase + off;
#pragma unroll
            for (int k = 0; k < NQ; ++k)
                dst.q[k] = *reinterpret_cast<const u32x4_t*>(kb + koff + k * 64);
        } else {
            const char* vb = vbase + off;
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

template <int D, int G, int DEPTH, int kChunk, bool QLDS, int W>
__global__ __launch_bounds__(64 * W) void decode_bf16_kernel(Params p) {
    bf16_item<D, G, DEPTH, kChunk, QLDS, W>(p, blockIdx.x);
}


// Shared prefix (parallel sampling, shared prompts): the leading tokens a group of
// sequences shares are read once for all of them. One wavefront per (group, KV head,
// partition of pre_tokens tokens); the M = members x G query rows of the group are the
// columns of the score tiles (set s holds rows 16 s .. 16 s + 15, zero past M), so each K
// and V tile feeds every member. Scores: v_mfma_f32_16x16x32_bf16, lane (r, c) then holds
// tokens r + 4i of query row 16 s + c; online softmax per column; PV:
// v_mfma_f32_16x16x16_bf16 with those probabilities (rounded to bf16) as A, leaving lane
// (r, c) with query rows 16 s + 4 r + i of output columns c * EV .. c * EV + EV - 1. Every
// (member, head) gets a partial record in slot `part`; the partition merge combines them
// with the members' own tokens.
template <int D, int NSET>
__device__ __forceinline__ void prefix_item(const Params& p, int id) {
    constexpr int ROW = D * 2;
    constexpr int NQ = D / 32;
    constexpr int WV = D / 8;
    constexpr int EV = D / 16;
    constexpr int DEPTH = 4;             // ring items: K and V of two groups
    constexpr int U = DEPTH / 2;
    static_assert(D == 64 || D == 128, "head size");

    const int lane = threadIdx.x & 63;
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
    const int G = p.Hq / p.Hkv;
    const int M = members * G;           // query rows (host checks M <= 16 * NSET)
    const int t0 = part * p.pre_tokens;
    if (first < 0 || first >= p.B || t0 >= shared_tok || members <= 0) return;
    const int ntok = min(p.pre_tokens, shared_tok - t0);
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
    auto goff = [&](int gq) -> int64_t {
        gq = gq < last ? gq : last;
        const int ph = __builtin_amdgcn_readlane(tblv, gq);
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
                        const float ai = __shfl(alpha, 4 * r + i);
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
__device__ __forceinline__ void multi_item(const Params& p, int id) {
    constexpr int ROW = D * 2;
    constexpr int NQ = D / 32;
    constexpr int WV = D / 8;
    constexpr int EV = D / 16;
    constexpr int DEPTH = 4;             // ring items: K and V of two groups
    constexpr int U = DEPTH / 2;
    static_assert(D == 64 || D == 128, "head size");

    const int lane = threadIdx.x & 63;
    // item order: KV head fastest (the heads spread over the XCDs), then query tile from
    // the last (a chunk's later tiles see the most tokens, so they start first), then
    // partition, then sequence: the tiles of one (sequence, KV head) run together on one
    // XCD and share its L2
    const int g = id % p.Hkv;
    int rest = id / p.Hkv;
    const int tile = p.n_tiles - 1 - rest % p.n_tiles;
    rest /= p.n_tiles;
    const int part = rest % p.n_parts;
    const int b = rest / p.n_parts;
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

    // scores of one group for every set: y[s][o + i] for tokens r + 4i of the group
    auto qk = [&](const Item& kit, float (&y)[NSET][8], int o) {
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NQ; ++k)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8_t, kit.q[k]),
                    __builtin_bit_cast(bf16x8_t, qf[s][k]), sc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) y[s][o + i] = sc[i] * cl2;
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
        uint32_t pw[NSET][4];
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            if (edge) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int tok = tg + (i >> 2) * 16 + r + 4 * (i & 3);
                    const bool ok = tok <= pos_c[s] && (i < 4 || live1);
                    y[s][i] = ok ? y[s][i] : -INFINITY;
                }
            }
            float mx = y[s][0];
#pragma unroll
            for (int i = 1; i < 8; ++i) mx = fmaxf(mx, y[s][i]);
            const float m_new = fmaxf(m_run[s], rows_max(mx));
            // a column that has seen no token yet keeps m = -inf: use 0 as its reference so
            // that its factors are exactly 0 instead of NaN
            const float m_ref = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run[s] - m_ref);   // per column
            m_run[s] = m_new;
            // rescale only when some column's maximum moved (a factor of 1 is exact)
            if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha, 4 * r + i);
#pragma unroll
                    for (int e = 0; e < EV; ++e) acc[s][e][i] *= ai;
                    lsum[s][i] *= ai;
                }
            }
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
#pragma unroll
        for (int w = 0; w < WV / 4; ++w) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t sel = h ? 0x07060302u : 0x05040100u;
                const u32x4_t bv = {__builtin_amdgcn_perm(vword(v0, 1, w), vword(v0, 0, w), sel),
                                    __builtin_amdgcn_perm(vword(v0, 3, w), vword(v0, 2, w), sel),
                                    __builtin_amdgcn_perm(vword(v1, 1, w), vword(v1, 0, w), sel),
                                    __builtin_amdgcn_perm(vword(v1, 3, w), vword(v1, 2, w), sel)};
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    const u32x4_t av = {pw[s][0], pw[s][1], pw[s][2], pw[s][3]};
                    acc[s][2 * w + h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, bv),
                        acc[s][2 * w + h], 0, 0, 0);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        issue_v(t + 2, v0);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(t + 3, v1);
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

// All multi-query items, four per 256-thread block.
template <int D, int NSET>
__global__ __launch_bounds__(256) void decode_multi_kernel(Params p) {
    const int item = blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (item < p.pre_items) multi_item<D, NSET>(p, item);
}

// The prefix partitions and the members' own tokens in one launch of 4-wave blocks, one
// item per wave: blocks below pre_blocks hold the prefix items (first, so that the longest
// work starts earliest), the rest the suffix partitions. A suffix partition is short (the
// tokens a member added after the shared prefix), so it gets a single wave and a small
// chunk, which starts its V loads after four K tiles rather than eight.
template <int D, int G, int NSET>
__global__ __launch_bounds__(256) void decode_shared_kernel(Params p) {
    const int bid = blockIdx.x;
    const int item = (bid < p.pre_blocks ? bid : bid - p.pre_blocks) * 4 + (int)(threadIdx.x >> 6);
    if (bid < p.pre_blocks) {
        if (item < p.pre_items) prefix_item<D, NSET>(p, item);
    } else if (item < p.suf_items) {
        bf16_item<D, G, PA_SHARED_DEPTH, PA_SHARED_CHUNK, false, 1>(p, item);
    }
}

// Combine the partitions of one (sequence, query head):
// out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i, with M = max_i m_i.
// Thread (pg, c4) folds partitions pg, pg + NPG, ... of float4 column c4, four per batch,
// rescaling its running sum when the maximum grows; the NPG partial sums then meet in
// LDS. The first batch is loaded before the partition count is known, together with the
// length (and group) that give it: slots below n_parts always lie in the row's workspace,
// and a slot past the count is dropped by a select, never weighted, since it may hold
// anything.
template <int D>
__global__ __launch_bounds__(256) void decode_reduce_kernel(Params p) {
    constexpr int C4 = D / 4;          // float4 columns
    constexpr int NPG = 256 / C4;      // partition groups per block
    __shared__ float4 red_o[NPG][C4];
    __shared__ float2 red_ml[NPG];

    const int h = blockIdx.x;
    const int y = blockIdx.y;          // the sequence, or in multi-query mode the query
    const int tid = threadIdx.x;
    const int c4 = tid % C4;
    const int pg = tid / C4;
    const int64_t row = (int64_t)y * p.Hq + h;
    const float2* ml = p.ws_ml + row * p.n_parts;
    const float* wo = p.ws_o + row * p.n_parts * D;
    float2 mlv[4];
    float4 ov[4];
    auto load_batch = [&](int i0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            int i = i0 + u * NPG;
            i = i < p.n_parts ? i : 0;
            mlv[u] = ml[i];
            ov[u] = reinterpret_cast<const float4*>(wo + (int64_t)i * D)[c4];
        }
    };
    load_batch(pg);

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
                for (int i = tid; i < D; i += 256) p.out[row * D + i] = 0.f;
                return;
            }
        } else {
            np = (L + p.part_tokens - 1) / p.part_tokens;
            if (np <= 1) return;
        }
    }

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float den = 0.f, m = -INFINITY;
    for (int i0 = pg; i0 < np; i0 += 4 * NPG) {
        if (i0 != pg) load_batch(i0);
        float mn = m;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (i0 + u * NPG < np) mn = fmaxf(mn, mlv[u].x);
        const float a = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first batch
        acc.x *= a; acc.y *= a; acc.z *= a; acc.w *= a;
        den *= a;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if (i0 + u * NPG < np) {
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
    red_o[pg][c4] = acc;
    if (c4 == 0) red_ml[pg] = make_float2(m, den);
    __syncthreads();
    if (pg == 0) {
        float M = red_ml[0].x;
#pragma unroll
        for (int j = 1; j < NPG; ++j) M = fmaxf(M, red_ml[j].x);
        float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
        float dsum = 0.f;
#pragma unroll
        for (int j = 0; j < NPG; ++j) {
            const float2 mlj = red_ml[j];
            const float w = __builtin_amdgcn_exp2f(mlj.x - M);   // 0 for a group with none
            const float4 x = red_o[j][c4];
            sum.x = fmaf(w, x.x, sum.x);
            sum.y = fmaf(w, x.y, sum.y);
            sum.z = fmaf(w, x.z, sum.z);
            sum.w = fmaf(w, x.w, sum.w);
            dsum = fmaf(w, mlj.y, dsum);
        }
        const float inv = 1.0f / dsum;
        reinterpret_cast<float4*>(p.out + row * D)[c4] =
            make_float4(sum.x * inv, sum.y * inv, sum.z * inv, sum.w * inv);
    }
}




// ---------------------------------------------------------------------------------------
// Stream decomposition (bf16 KV). The rows (sequence b, KV head g), each cut into
// ceil(L_b / 16) groups of 16 tokens, are laid end to end into one stream of T groups,
// and each of nw resident waves takes an equal contiguous slice of it. A wave walks its
// slice with one load ring that never drains between rows: it finishes rows it covers
// whole by writing the output directly, and leaves a partial state (max, sum, unscaled
// output) for the at most two rows it covers only in part; stream_reduce_kernel merges
// those. Each group's K tile and V tile are 4 KiB items of the ring; the online softmax
// is updated once per group. Block-table lookups for 64 groups at a time ("window") are
// resolved lane-parallel: lane i finds the row of group sw + i by a binary search over
// the per-sequence prefix of group counts kept in LDS, then gathers its table entry.
// SPLIT: blocks of 8 tokens, so a 16-token group spans two physical blocks; each group
// then has two tile offsets (tokens 0-7 and 8-15) and K lanes / V loads pick theirs.
template <int D, int G, int DEPTH, bool SPLIT>
__global__ __launch_bounds__(256) void decode_stream_kernel(Params p) {
    constexpr int ROW = D * 2;              // bytes per cached row
    constexpr int NQ = D / 32;              // 16-byte registers per ring item
    constexpr int WV = D / 8;               // bytes of a V row per lane per load (16 or 8)
    constexpr int EV = D / 16;              // bf16 elements per lane per V load
    constexpr int NSET = (G + 3) / 4;       // head sets of 4
    constexpr int G4 = G < 4 ? G : 4;       // distinct heads in a set
    constexpr int U = DEPTH / 2;            // groups in flight ahead of the consumer
    static_assert(D == 64 || D == 128, "head size");
    static_assert(DEPTH >= 2 && DEPTH % 2 == 0, "ring holds whole groups (K and V)");

    extern __shared__ int lds_prefix[];
    int* Cs = lds_prefix;           // [B + 1] exclusive prefix of groups per sequence
    int* Ls = lds_prefix + p.B + 1; // [B] lengths clamped into the table's capacity
    __shared__ int wsum[4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int cap = p.max_blocks * p.bs;

    // ---- groups per sequence and their exclusive prefix over the batch (whole block)
    const int per = (p.B + 255) >> 8;
    int loc = 0;
    for (int i = 0; i < per; ++i) {
        const int bb = tid * per + i;
        if (bb < p.B) {
            int L = p.lens[bb];
            L = L < 0 ? 0 : (L > cap ? cap : L);
            Ls[bb] = L;
            loc += (L + 15) >> 4;
        }
    }
    int inc = loc;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(inc, d);
        if (lane >= d) inc += y;
    }
    if (lane == 63) wsum[wid] = inc;
    __syncthreads();
    int run = inc - loc;
    for (int v = 0; v < wid; ++v) run += wsum[v];
    for (int i = 0; i < per; ++i) {
        const int bb = tid * per + i;
        if (bb < p.B) {
            Cs[bb] = run;
            run += (Ls[bb] + 15) >> 4;
        }
    }
    if (tid == 255) Cs[p.B] = run;
    __syncthreads();

    const int T = __builtin_amdgcn_readfirstlane(Cs[p.B]) * p.Hkv;
    const int gw = blockIdx.x * 4 + wid;
    int nwe = T / p.min_slice;
    nwe = nwe < 1 ? 1 : (nwe > p.nw ? p.nw : nwe);
    if (T == 0) nwe = 0;
    if (gw == 0 && lane == 0) {
        p.meta[0] = T;
        p.meta[1] = nwe;
    }
    // empty sequences: a zero row per query head
    for (int bb = gw; bb < p.B; bb += p.nw) {
        if (__builtin_amdgcn_readfirstlane(Ls[bb]) == 0) {
            float* o = p.out + (int64_t)bb * p.Hq * D;
            for (int i = lane; i < p.Hq * D; i += 64) o[i] = 0.f;
        }
    }
    if (gw >= nwe) return;
    const int s0 = (int)((int64_t)gw * T / nwe);
    const int s1 = (int)((int64_t)(gw + 1) * T / nwe);
    const int ns = s1 - s0;

    const int64_t tile_bytes = (int64_t)p.bs * ROW;              // one (block, head) tile
    const int64_t blk_bytes = (int64_t)p.Hkv * tile_bytes;       // one physical block
    const int bs_mask = p.bs - 1;

    // ---- window: lane i describes group sw + i of the slice (clamped into it)
    uint32_t w_lo = 0, w_hi = 0;   // byte offset of the group's tile in either cache
    uint32_t w_lo1 = 0, w_hi1 = 0; // SPLIT: offset of the tile holding tokens 8-15
    int w_row = 0, w_j = 0;        // its row (b * Hkv + g) and group within the row
    int sw = s0;
    auto window = [&](int base) {
        int s = base + lane;
        s = s < s1 ? s : s1 - 1;
        int lo = 0, hi = p.B - 1;
        while (lo < hi) {           // first sequence whose groups end past s
            const int mid = (lo + hi) >> 1;
            if (Cs[mid + 1] * p.Hkv > s) hi = mid;
            else lo = mid + 1;
        }
        const int n = Cs[lo + 1] - Cs[lo];
        const int off = s - Cs[lo] * p.Hkv;
        const int g = off / n;
        const int j = off - g * n;
        const int32_t* trow = p.tables + (int64_t)lo * p.max_blocks;
        int e = trow[(j << 4) >> p.bs_shift];
        e = e < 0 ? 0 : (e >= p.num_blocks ? p.num_blocks - 1 : e);
        const int64_t o = (int64_t)e * blk_bytes + (int64_t)g * tile_bytes +
                          (int64_t)((j << 4) & bs_mask) * ROW;
        w_lo = (uint32_t)o;
        w_hi = (uint32_t)((uint64_t)o >> 32);
        if constexpr (SPLIT) {     // the second block of the group (clamped into the row)
            int i1 = 2 * j + 1;
            i1 = i1 < p.max_blocks ? i1 : p.max_blocks - 1;
            int e1 = trow[i1];
            e1 = e1 < 0 ? 0 : (e1 >= p.num_blocks ? p.num_blocks - 1 : e1);
            const int64_t o1 = (int64_t)e1 * blk_bytes + (int64_t)g * tile_bytes;
            w_lo1 = (uint32_t)o1;
            w_hi1 = (uint32_t)((uint64_t)o1 >> 32);
        }
        w_row = lo * p.Hkv + g;
        w_j = j;
    };
    window(sw);

    // ---- consumer cursor (wave-uniform, kept in scalar registers): sequence, KV head,
    // group in row, groups in row, tokens in row. Lengths are re-read through the scalar
    // cache so that no vector register enters the cursor's updates.
    typedef __attribute__((address_space(4))) const int32_t* const_i32p;
    const const_i32p slens = (const_i32p)(p.lens);
    auto seq_len = [&](int bb) -> int {
        const int L = slens[bb];
        return L < 0 ? 0 : (L > cap ? cap : L);
    };
    const int row0 = __builtin_amdgcn_readlane(w_row, 0);
    int cb = row0 / p.Hkv;
    int cg = row0 - cb * p.Hkv;
    int cj = __builtin_amdgcn_readlane(w_j, 0);
    int cL = seq_len(cb);
    int cn = (cL + 15) >> 4;
    if (lane == 0) p.desc[gw] = make_int4(cb, cg, s0 - cj, cn);

    const int r = lane >> 4;     // row group
    const int c = lane & 15;     // column
    // query fragments of the current row and of the next row the loads reach
    u32x4_t qf[NSET][NQ], qn[NSET][NQ];
    auto load_q = [&](int row, u32x4_t (&dst)[NSET][NQ]) {
        const int bq = row / p.Hkv;
        const int gq = row - bq * p.Hkv;
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            const int h = 4 * s + ((c & 3) % G4);
            const char* qrow = p.q + ((int64_t)bq * p.Hq + gq * G + h) * ROW;
#pragma unroll
            for (int k = 0; k < NQ; ++k)
                dst[s][k] = *reinterpret_cast<const u32x4_t*>(qrow + (k * 32 + r * 8) * 2);
        }
    };
    load_q(row0, qf);
#pragma unroll
    for (int s = 0; s < NSET; ++s)
#pragma unroll
        for (int k = 0; k < NQ; ++k) qn[s][k] = qf[s][k];
    int qn_row = -1;       // row whose fragments sit in qn
    int iss_row = row0;    // row of the last K tile issued

    // K: lane c of a row group feeds token (c / 4) + 4 (c % 4) of the group; with SPLIT,
    // tokens 8-15 (c % 4 >= 2) come from the second block, at row token - 8
    const int ktok = (c >> 2) + 4 * (c & 3);
    const bool khi = SPLIT && ktok >= 8;
    const uint32_t koff = (uint32_t)((SPLIT ? (ktok & 7) : ktok) * ROW + r * 16);
    const uint32_t voff = (uint32_t)(r * ROW + c * WV);
    struct Item {
        u32x4_t q[NQ];
    };
    auto tile_off = [&](int gq) -> uint64_t {
        int s = s0 + gq;
        s = s < s1 ? s : s1 - 1;
        if (s - sw >= 64) {
            sw += 64;
            window(sw);
        }
        const int idx = s - sw;
        return ((uint64_t)__builtin_amdgcn_readlane(w_hi, idx) << 32) |
               (uint64_t)__builtin_amdgcn_readlane(w_lo, idx);
    };
    // SPLIT: the second block's tile of the same group (the window is already in place)
    auto tile_off1 = [&](int gq) -> uint64_t {
        int s = s0 + gq;
        s = s < s1 ? s : s1 - 1;
        const int idx = s - sw;
        return ((uint64_t)__builtin_amdgcn_readlane(w_hi1, idx) << 32) |
               (uint64_t)__builtin_amdgcn_readlane(w_lo1, idx);
    };
    auto issue_k = [&](int gq, Item& dst) {
        const uint64_t off = tile_off(gq);
        int s = s0 + gq;
        s = s < s1 ? s : s1 - 1;
        const int row = __builtin_amdgcn_readlane(w_row, s - sw);
        if (row != iss_row) {       // the loads enter a new row: fetch its query early
            iss_row = row;
            qn_row = row;
            load_q(row, qn);
        }
        const char* kb = p.k + off;
        if constexpr (SPLIT) {
            const char* kb1 = p.k + tile_off1(gq);
            kb = khi ? kb1 : kb;
        }
#pragma unroll
        for (int k = 0; k < NQ; ++k)
            dst.q[k] = *reinterpret_cast<const u32x4_t*>(kb + koff + k * 64);
    };
    // V load k holds rows r + 4k; with SPLIT, loads 2 and 3 (rows 8-15) read the second
    // block at rows r + 4 (k - 2)
    auto issue_v = [&](int gq, Item& dst) {
        const char* vb = p.v + tile_off(gq);
        const char* vb1 = vb + 2 * 4 * ROW;
        if constexpr (SPLIT) vb1 = p.v + tile_off1(gq);
        // address of V load k (rows r + 4k of the group)
        auto vaddr = [&](int k) -> const char* {
            return k < 2 ? vb + voff + k * 4 * ROW : vb1 + voff + (k - 2) * 4 * ROW;
        };
        if constexpr (WV == 16) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                dst.q[k] = *reinterpret_cast<const u32x4_t*>(vaddr(k));
        } else {
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                const u32x2_t a = *reinterpret_cast<const u32x2_t*>(vaddr(k));
                const u32x2_t e = *reinterpret_cast<const u32x2_t*>(vaddr(k + 1));
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
    auto reset = [&]() {
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            m_run[s] = -INFINITY;
            l_run[s] = 0.f;
#pragma unroll
            for (int e = 0; e < EV; ++e) acc[s][e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    };
    reset();
    bool first_seg = true;   // the slice's first row segment
    int seg_j0 = cj;         // first group of the current row segment
    const float cl2 = p.scale_log2;

    // write the state of the current row segment: the output if the segment is the whole
    // row, else a partial record (slot 0: the slice's first segment, slot 1: its last)
    auto flush = [&]() {
        const bool whole = seg_j0 == 0 && cj == cn - 1;
        float lh[NSET][4], mh[NSET][4];
#pragma unroll
        for (int s = 0; s < NSET; ++s) {
            l_run[s] = rows_sum(l_run[s]);   // the output tile needs no sum: rows repeat
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                lh[s][m] = quad_bcast(l_run[s], m);
                mh[s][m] = quad_bcast(m_run[s], m);
            }
        }
        if (r == 0) {
            const int rec = 2 * gw + (first_seg ? 0 : 1);
#pragma unroll
            for (int s = 0; s < NSET; ++s) {
#pragma unroll
                for (int m = 0; m < G4; ++m) {
                    const int h = 4 * s + m;
                    if (whole) {
                        const float inv = 1.0f / lh[s][m];
                        float* dst = p.out + ((int64_t)cb * p.Hq + cg * G + h) * D + c * EV;
#pragma unroll
                        for (int e = 0; e < EV; e += 4)
                            *reinterpret_cast<float4*>(dst + e) =
                                make_float4(acc[s][e][m] * inv, acc[s][e + 1][m] * inv,
                                            acc[s][e + 2][m] * inv, acc[s][e + 3][m] * inv);
                    } else {
                        float* dst = p.rec_o + ((int64_t)rec * G + h) * D + c * EV;
#pragma unroll
                        for (int e = 0; e < EV; e += 4)
                            *reinterpret_cast<float4*>(dst + e) =
                                make_float4(acc[s][e][m], acc[s][e + 1][m], acc[s][e + 2][m], acc[s][e + 3][m]);
                        if (c == 0) p.rec_ml[(int64_t)rec * G + h] = make_float2(mh[s][m], lh[s][m]);
                    }
                }
            }
        }
    };

    Item ring[DEPTH];
#pragma unroll
    for (int u = 0; u < U; ++u) {   // fill the ring in stream order (the waits count on it)
        __builtin_amdgcn_sched_barrier(0);
        issue_k(u, ring[2 * u]);
        __builtin_amdgcn_sched_barrier(0);
        issue_v(u, ring[2 * u + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);

    for (int t0 = 0; t0 < ns; t0 += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + u;
            Item& kit = ring[2 * u];
            Item& vit = ring[2 * u + 1];
            const bool live = t < ns;
            const int valid = min(16, cL - 16 * cj);   // tokens of the group (last may be short)
            float y[NSET][4];
            uint32_t pw[NSET][2];   // bf16 probabilities of tokens r + 4i, two per dword
            if (live) {
                // ---- scores of the group on the matrix cores, in log2 units
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
                // ---- online softmax update: lane holds tokens r + 4i of head column c
#pragma unroll
                for (int s = 0; s < NSET; ++s) {
                    if (valid < 16) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) y[s][i] = (r + 4 * i < valid) ? y[s][i] : -INFINITY;
                    }
                    const float mx = fmaxf(fmaxf(y[s][0], y[s][1]), fmaxf(y[s][2], y[s][3]));
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
                    // probabilities, rounded to bf16 for the matrix cores; the sum takes
                    // the rounded values too, so the weights it divides by are the ones used
                    const bf16x2_t p01 = __builtin_convertvector(
                        (f32x2_t){__builtin_amdgcn_exp2f(y[s][0] - m_new), __builtin_amdgcn_exp2f(y[s][1] - m_new)}, bf16x2_t);
                    const bf16x2_t p23 = __builtin_convertvector(
                        (f32x2_t){__builtin_amdgcn_exp2f(y[s][2] - m_new), __builtin_amdgcn_exp2f(y[s][3] - m_new)}, bf16x2_t);
                    pw[s][0] = __builtin_bit_cast(uint32_t, p01);
                    pw[s][1] = __builtin_bit_cast(uint32_t, p23);
                    l_run[s] = l_run[s] * alpha + ((lo_bf16(pw[s][0]) + hi_bf16(pw[s][0])) +
                                                   (lo_bf16(pw[s][1]) + hi_bf16(pw[s][1])));
                }
                // ---- o += p * V on the matrix cores; V rows past the end may hold anything
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
                // One v_mfma_f32_16x16x16_bf16 per output column set e: A = the lane's four
                // probabilities (row = head column c, k = tokens r + 4i, exactly as the score
                // tile left them), B = V[r + 4i][c * EV + e], gathered from the four V loads
                // with byte permutes. Output rows 4r..4r+3 repeat the G4 heads for every r.
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
            if (live) {
                const bool seg_end = cj == cn - 1 || t == ns - 1;
                const int cj_next = seg_end ? 0 : cj + 1;   // defined on every path
                if (seg_end) {
                    flush();
                    if (t < ns - 1) {     // the slice goes on into the next row
                        ++cg;
                        if (cg == p.Hkv) {
                            cg = 0;
                            do {   // skip empty sequences (bounded by the batch)
                                cL = seq_len(++cb);
                            } while (cL == 0 && cb < p.B - 1);
                        }
                        cn = (cL + 15) >> 4;
                        seg_j0 = 0;
                        first_seg = false;
                        const int row = cb * p.Hkv + cg;
                        // The prefetched fragments are copied (the compiler waits for
                        // exactly their loads); fragments loaded here are waited for at
                        // once (a rare case), so that past this point the query
                        // registers hold no pending load on any path and the ring's
                        // waits stay exact.
                        if (qn_row == row) {
#pragma unroll
                            for (int s = 0; s < NSET; ++s)
#pragma unroll
                                for (int k = 0; k < NQ; ++k) qf[s][k] = qn[s][k];
                        } else {
                            load_q(row, qf);
                            __builtin_amdgcn_s_waitcnt(kWaitVm0);
                        }
                        reset();
                    }
                }
                cj = cj_next;
            }
        }
    }
}

// Merge the partial records of rows that cross slice boundaries. Group w looks at the
// row holding the first group of slice w; it merges it only when that row began inside
// slice w - 1, so every split row is merged exactly once, records in slice order. The
// merge is latency-bound: one thread per float4 of the row's G x D output, the header
// and the descriptor fetched together, and a row's records loaded kBatch at a time.
template <int D, int G>
__global__ __launch_bounds__(G * D / 4 < 64 ? 64 : G * D / 4) void stream_reduce_kernel(Params p) {
    constexpr int C4 = D / 4;
    constexpr int kBatch = 8;
    const int w = blockIdx.x;
    const int T = p.meta[0];
    const int nwe = p.meta[1];
    const int4 d = p.desc[w];          // b, g, row start, row groups
    if (w == 0 || w >= nwe) return;
    const int s0w = (int)((int64_t)w * T / nwe);
    if (d.z >= s0w) return;            // the row starts in slice w: not split here
    const int s0p = (int)((int64_t)(w - 1) * T / nwe);
    if (d.z < s0p) return;             // began before slice w - 1: merged by an earlier group
    const int i = threadIdx.x;
    if (i >= G * C4) return;
    const int h = i / C4, c4 = i % C4;
    const int last = d.z + d.w - 1;
    const int wb = (int)(((int64_t)(last + 1) * nwe - 1) / T);   // slice holding the last group
    const int nrec = wb - w + 2;       // slices w - 1 .. wb
    const int rec_a = 2 * (w - 1) + (d.z == s0p ? 0 : 1);
    float M = -INFINITY, l = 0.f;
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int x0 = 0; x0 < nrec; x0 += kBatch) {   // running merge in slice order
        float2 ml[kBatch];
        float4 v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const int x = x0 + k < nrec ? x0 + k : nrec - 1;
            const int rec = x == 0 ? rec_a : 2 * (w - 1 + x);
            ml[k] = p.rec_ml[(int64_t)rec * G + h];
            v[k] = reinterpret_cast<const float4*>(p.rec_o + ((int64_t)rec * G + h) * D)[c4];
        }
        float Mb = M;
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
            if (x0 + k < nrec) Mb = fmaxf(Mb, ml[k].x);
        const float a = __builtin_amdgcn_exp2f(M - Mb);   // 0 on the first batch
        o.x *= a; o.y *= a; o.z *= a; o.w *= a;
        l *= a;
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            if (x0 + k < nrec) {
                const float wgt = __builtin_amdgcn_exp2f(ml[k].x - Mb);
                o.x += wgt * v[k].x; o.y += wgt * v[k].y; o.z += wgt * v[k].z; o.w += wgt * v[k].w;
                l += wgt * ml[k].y;
            }
        }
        M = Mb;
    }
    const float inv = 1.0f / l;
    reinterpret_cast<float4*>(p.out + ((int64_t)d.x * p.Hq + d.y * G + h) * D)[c4] =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
}

template <bool BF16, int D, int G>
hipError_t launch_one(const Params& prm, int B, int Hkv, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if constexpr (BF16) {
        hipLaunchKernelGGL((decode_bf16_kernel<D, G, PA_BF16_DEPTH, PA_BF16_CHUNK, (PA_BF16_QLDS != 0), PA_BF16_WAVES>),
                           dim3(prm.n_parts * Hkv * B), dim3(64 * PA_BF16_WAVES), 0, s, prm);
    } else {
        const size_t lds = (size_t)prm.part_tokens * G * sizeof(float) +
                           (size_t)(prm.part_tokens / 16) * sizeof(int);
        hipLaunchKernelGGL((decode_partition_kernel<BF16, D, G, PA_DECODE_DEPTH>),
                           dim3(prm.n_parts * Hkv * B), dim3(64), lds, s, prm);
    }
    if (prm.n_parts > 1)
        hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(prm.Hq, B), dim3(256), 0, s, prm);
    return hipGetLastError();
}

// Launch shape of the stream kernel on the current device: one 4-wave workgroup per CU,
// so every SIMD runs exactly one wave (two waves sharing a SIMD are served very unevenly:
// the older one starves the younger, and equal slices then finish far apart). The
// workgroup reserves just over half of a CU's LDS, which makes that placement certain.
// Cached per device.
int stream_shape(size_t need_lds, int* nw, size_t* lds) {
    struct Entry {
        int dev, cus;
        size_t half;
    };
    static std::mutex mu;
    static Entry cache[16];
    static int used = 0;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    Entry en{-1, 0, 0};
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].dev == dev) en = cache[i];
    }
    if (en.dev < 0) {
        int cus = 0, per_cu = 0, per_block = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return (int)e;
        e = hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev);
        if (e != hipSuccess) return (int)e;
        e = hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (e != hipSuccess) return (int)e;
        size_t half = (size_t)per_cu / 2 + 1024;
        if (half > (size_t)per_block) half = 0;   // cannot force it: rely on even dispatch
        en = Entry{dev, cus, half};
        std::lock_guard<std::mutex> lock(mu);
        if (used < 16) cache[used++] = en;
    }
    *nw = en.cus * 4;
    *lds = need_lds > en.half ? need_lds : en.half;
    return 0;
}

template <int D, int G, bool SPLIT>
hipError_t launch_stream(Params prm, int nw_req, void* stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    size_t lds = (size_t)(2 * prm.B + 1) * sizeof(int);
    int nw = nw_req;
    if (nw <= 0) {
        const int e = stream_shape(lds, &nw, &lds);
        if (e != 0) return (hipError_t)e;
    }
    nw = nw > pa_internal::kMaxStreamWaves ? pa_internal::kMaxStreamWaves : nw;
    nw = (nw + 3) / 4 * 4;
    prm.nw = nw;
    hipLaunchKernelGGL((decode_stream_kernel<D, G, PA_STREAM_DEPTH, SPLIT>), dim3(nw / 4), dim3(256), lds, s, prm);
    constexpr int kMergeThreads = G * D / 4 < 64 ? 64 : G * D / 4;
    hipLaunchKernelGGL((stream_reduce_kernel<D, G>), dim3(nw), dim3(kMergeThreads), 0, s, prm);
    return hipGetLastError();
}

template <int D, bool SPLIT>
hipError_t dispatch_stream_g(const Params& prm, int G, int nw, void* stream) {
    switch (G) {
        case 1: return launch_stream<D, 1, SPLIT>(prm, nw, stream);
        case 2: return launch_stream<D, 2, SPLIT>(prm, nw, stream);
        case 4: return launch_stream<D, 4, SPLIT>(prm, nw, stream);
        case 8: return launch_stream<D, 8, SPLIT>(prm, nw, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16, int D>
hipError_t dispatch_g(const Params& prm, int B, int Hkv, int G, void* stream) {
    switch (G) {
        case 1: return launch_one<BF16, D, 1>(prm, B, Hkv, stream);
        case 2: return launch_one<BF16, D, 2>(prm, B, Hkv, stream);
        case 4: return launch_one<BF16, D, 4>(prm, B, Hkv, stream);
        case 8: return launch_one<BF16, D, 8>(prm, B, Hkv, stream);
        default: return hipErrorInvalidValue;
    }
}

template <bool BF16>
hipError_t dispatch_d(const Params& prm, int B, int Hkv, int D, int G, void* stream) {
    if (D == 64) return dispatch_g<BF16, 64>(prm, B, Hkv, G, stream);
    if (D == 128) return dispatch_g<BF16, 128>(prm, B, Hkv, G, stream);
    return hipErrorInvalidValue;
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
    hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(prm.Hq, prm.B), dim3(256), 0, s, prm);
    return hipGetLastError();
}

template <int D>
hipError_t launch_multi_d(const Params& prm, int nset, hipStream_t s) {
    const dim3 grid((prm.pre_items + 3) / 4);
    if (nset == 1) hipLaunchKernelGGL((decode_multi_kernel<D, 1>), grid, dim3(256), 0, s, prm);
    else if (nset == 2) hipLaunchKernelGGL((decode_multi_kernel<D, 2>), grid, dim3(256), 0, s, prm);
    else hipLaunchKernelGGL((decode_multi_kernel<D, 4>), grid, dim3(256), 0, s, prm);
    if (prm.n_parts > 1)
        hipLaunchKernelGGL((decode_reduce_kernel<D>), dim3(prm.Hq, prm.total_q), dim3(256), 0, s, prm);
    return hipGetLastError();
}

}  // namespace

namespace pa_internal {

int launch_decode(const DecodeLaunch& a, const char** err) {
    Params prm{};   // zero: no shared-prefix groups, no stream records
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
    (void)kLog2e;
    prm.rec_o = a.rec_o;
    prm.rec_ml = reinterpret_cast<float2*>(a.rec_ml);
    prm.desc = reinterpret_cast<int4*>(a.desc);
    prm.meta = a.meta;
    prm.nw = 0;
    prm.min_slice = a.min_slice > 0 ? a.min_slice : 1;
    if (a.B == 0) return 0;
    const int G = a.Hq / a.Hkv;
    hipError_t e;
    if (a.path == kPathStream) {
        const bool split = a.bs < 16;
        e = a.D == 64 ? (split ? dispatch_stream_g<64, true>(prm, G, a.stream_waves, a.stream)
                               : dispatch_stream_g<64, false>(prm, G, a.stream_waves, a.stream))
          : a.D == 128 ? (split ? dispatch_stream_g<128, true>(prm, G, a.stream_waves, a.stream)
                                : dispatch_stream_g<128, false>(prm, G, a.stream_waves, a.stream))
                       : hipErrorInvalidValue;
    } else {
        e = a.kv_dtype == 1 ? dispatch_d<true>(prm, a.B, a.Hkv, a.D, G, a.stream)
                            : dispatch_d<false>(prm, a.B, a.Hkv, a.D, G, a.stream);
    }
    if (e != hipSuccess) {
        *err = hipGetErrorString(e);
        return (int)e;
    }
    return 0;
}

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
